// Shared device/host helpers of the gfx950 drafter engine.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e3 {

constexpr int kWave = 64;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// round-to-nearest-even; NaN kept quiet
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// 8 bf16 (one 16-byte load) dotted with 8 fp32 values
__device__ __forceinline__ float dot8(const uint4 w, const float4 a, const float4 b, float acc) {
  acc = fmaf(bf16_lo(w.x), a.x, acc);
  acc = fmaf(bf16_hi(w.x), a.y, acc);
  acc = fmaf(bf16_lo(w.y), a.z, acc);
  acc = fmaf(bf16_hi(w.y), a.w, acc);
  acc = fmaf(bf16_lo(w.z), b.x, acc);
  acc = fmaf(bf16_hi(w.z), b.y, acc);
  acc = fmaf(bf16_lo(w.w), b.z, acc);
  acc = fmaf(bf16_hi(w.w), b.w, acc);
  return acc;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// streaming (read-once) 16-byte load of weights
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- wave / block reductions -------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// DPP lane moves (VALU, no LDS): control codes of the gfx9 encoding
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]: lane i <- i ^ 1
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]: lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8-lane half row
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within each 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of L consecutive lanes (L a power of two up to 64);
// every lane of a group gets the same bits (each step adds a lane's value to its
// partner's, the partner adding the same two values).  Up to 16 lanes in DPP moves.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "power-of-two lane group");
  if constexpr (L >= 2) v += dpp_move<kDppQuadSwap1>(v);
  if constexpr (L >= 4) v += dpp_move<kDppQuadSwap2>(v);
  if constexpr (L >= 8) v += dpp_move<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp_move<kDppMirror>(v);
  if constexpr (L >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Reduce-scatter over the wave of NV values per lane (NV a power of two, 2..32):
// afterwards the 64 / NV consecutive lanes from j * 64 / NV on hold, in v[0], the
// wave's sum of value j.  Each halving step trades half of the remaining values with
// a partner lane whose index differs in one more bit and keeps the half that bit
// selects; the bits left over are then summed whole.  That is NV - 1 + 6 - log2 NV
// exchanges instead of 6 NV, and the ones inside 16 lanes are DPP moves.  The
// partners for bits 2 and 3 are lane ^ 7 and lane ^ 15 (the DPP mirrors): they still
// flip the bit being split and share every bit already split, and the masks used
// span all 64 lanes, so each lane's value is counted once.
template <int O>
__device__ __forceinline__ float lane_exchange(float v) {
  if constexpr (O == 1) return dpp_move<kDppQuadSwap1>(v);
  else if constexpr (O == 2) return dpp_move<kDppQuadSwap2>(v);
  else if constexpr (O == 4) return dpp_move<kDppHalfMirror>(v);  // partner lane ^ 7
  else if constexpr (O == 8) return dpp_move<kDppMirror>(v);      // partner lane ^ 15
  else return __shfl_xor(v, O, kWave);
}

template <int O, int NV>
__device__ __forceinline__ void rs_step(float (&v)[32], int lane) {
  constexpr int H = NV / 2;
  const bool upper = (lane & O) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = upper ? v[i] : v[i + H];
    const float keep = upper ? v[i + H] : v[i];
    v[i] = keep + lane_exchange<O>(send);
  }
}

template <int NV>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[32]) {
  static_assert(NV >= 2 && NV <= 32 && (NV & (NV - 1)) == 0, "2..32 values, a power of two");
  const int lane = threadIdx.x & 63;
  // halving steps on lane bits 5, 4, ... until one value is left per lane
  if constexpr (NV >= 32) rs_step<32, 32>(v, lane);
  if constexpr (NV >= 16) rs_step<(NV >= 32 ? 16 : 32), 16>(v, lane);
  if constexpr (NV >= 8) rs_step<(NV >= 32 ? 8 : NV >= 16 ? 16 : 32), 8>(v, lane);
  if constexpr (NV >= 4) rs_step<(NV >= 32 ? 4 : NV >= 16 ? 8 : NV >= 8 ? 16 : 32), 4>(v, lane);
  rs_step<(NV >= 32 ? 2 : NV >= 16 ? 4 : NV >= 8 ? 8 : NV >= 4 ? 16 : 32), 2>(v, lane);
  // the remaining lane bits are summed whole
  constexpr int used = NV >= 32 ? 5 : NV >= 16 ? 4 : NV >= 8 ? 3 : NV >= 4 ? 2 : 1;  // bits 5.. consumed
  if constexpr (used < 5) v[0] += lane_exchange<(used == 1 ? 16 : used == 2 ? 8 : used == 3 ? 4 : 2)>(v[0]);
  if constexpr (used < 4) v[0] += lane_exchange<(used == 1 ? 8 : used == 2 ? 4 : 2)>(v[0]);
  if constexpr (used < 3) v[0] += lane_exchange<(used == 1 ? 4 : 2)>(v[0]);
  if constexpr (used < 2) v[0] += lane_exchange<2>(v[0]);
  v[0] += lane_exchange<1>(v[0]);
}

// sum of `count` per-block partial sums (this thread's share)
__device__ __forceinline__ float sum_partials(const float* __restrict__ p, int count) {
  float s = 0.f;
  for (int i = threadIdx.x; i < count; i += blockDim.x) s += p[i];
  return s;
}

// sum over the block of two values; `red` is LDS with room for 2 * waves floats.
// Every thread gets the totals.  NT: the block's thread count when known at compile
// time (blockDim.x is a memory load, whose wait would also wait for every load
// issued before it).
template <int NT = 0>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (NT ? NT : int(blockDim.x)) >> 6;
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane == 0) { red[w] = a; red[nw + w] = b; }
  __syncthreads();
  a = 0.f; b = 0.f;
  for (int i = 0; i < nw; ++i) { a += red[i]; b += red[nw + i]; }
  __syncthreads();
}

// (value, index) pair compare: larger value wins, lower index wins a tie
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// s_waitcnt vmcnt(N), the other counters untouched
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int kArgmaxBatch = 8;  // candidate loads per thread in flight together

// One thread's batch of argmax candidates: kArgmaxBatch (value, index, carried
// value) triples, strided by the block size from b0.
struct ArgmaxBatch {
  float v[kArgmaxBatch];
  int ix[kArgmaxBatch], t[kArgmaxBatch];
};

template <int NT = 0>
__device__ __forceinline__ void argmax_load(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                            const int32_t* __restrict__ pt, int count, int b0,
                                            ArgmaxBatch& c) {
#pragma unroll
  for (int j = 0; j < kArgmaxBatch; ++j) {
    const int b = b0 + int(threadIdx.x) + j * (NT ? NT : int(blockDim.x));
    const bool in = b < count;
    c.v[j] = in ? pv[b] : -INFINITY;
    c.ix[j] = in ? pi[b] : 0x7FFFFFFF;
    c.t[j] = (in && pt) ? pt[b] : 0;
  }
}

// Argmax over `count` (value, index) candidates, the lower index winning a tie;
// every thread gets the winning index.  When pt is given, pt[c] is a value
// carried with candidate c and *tok receives the winner's.  Each thread's
// candidates are loaded kArgmaxBatch at a time, so a block of T threads covers
// kArgmaxBatch * T candidates per memory round trip; `first` is the batch from
// 0, already loaded by argmax_load (a caller can issue it ahead of other loads).
// sv/si/st: LDS, one slot per wave (st only read when pt is given).  MORE = false:
// the caller guarantees count <= kArgmaxBatch * blockDim.x (no further batches,
// and no loop, whose loads would make the compiler wait for every load in flight).
// NT: the block's thread count when known at compile time (as block_sum2).
template <bool MORE = true, int NT = 0>
__device__ __forceinline__ int block_argmax_from(const ArgmaxBatch& first, const float* __restrict__ pv,
                                                 const int32_t* __restrict__ pi,
                                                 const int32_t* __restrict__ pt, int count, float* sv,
                                                 int* si, int* st, int* tok) {
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF, bt = 0;
#pragma unroll
  for (int j = 0; j < kArgmaxBatch; ++j)
    if (better(first.v[j], first.ix[j], bv, bi)) { bv = first.v[j]; bi = first.ix[j]; bt = first.t[j]; }
  if constexpr (MORE)
  for (int b0 = kArgmaxBatch * int(blockDim.x); b0 < count; b0 += kArgmaxBatch * int(blockDim.x)) {
    ArgmaxBatch c;
    argmax_load(pv, pi, pt, count, b0, c);
#pragma unroll
    for (int j = 0; j < kArgmaxBatch; ++j)
      if (better(c.v[j], c.ix[j], bv, bi)) { bv = c.v[j]; bi = c.ix[j]; bt = c.t[j]; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    const int ot = __shfl_xor(bt, o, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; bt = ot; }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (NT ? NT : int(blockDim.x)) >> 6;
  if (lane == 0) {
    sv[w] = bv;
    si[w] = bi;
    if (pt) st[w] = bt;
  }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
  if (pt) bt = st[0];
  for (int k = 1; k < nw; ++k)
    if (better(sv[k], si[k], bv, bi)) {
      bv = sv[k];
      bi = si[k];
      if (pt) bt = st[k];
    }
  __syncthreads();
  if (tok) *tok = bt;
  return bi;
}

__device__ __forceinline__ int block_argmax_carry(const float* __restrict__ pv,
                                                  const int32_t* __restrict__ pi,
                                                  const int32_t* __restrict__ pt, int count,
                                                  float* sv, int* si, int* st, int* tok) {
  ArgmaxBatch c;
  argmax_load(pv, pi, pt, count, 0, c);
  return block_argmax_from(c, pv, pi, pt, count, sv, si, st, tok);
}

__device__ __forceinline__ int block_argmax(const float* __restrict__ pv,
                                            const int32_t* __restrict__ pi, int count,
                                            float* sv, int* si) {
  return block_argmax_carry(pv, pi, nullptr, count, sv, si, nullptr, nullptr);
}

// cos/sin of pos * inv_freq, the angle reduced modulo 2*pi in double first
__device__ __forceinline__ void rope_cs(int pos, double inv_freq, float* c, float* s) {
  const double twopi = 6.283185307179586476925286766559;
  double a = double(pos) * inv_freq;
  a -= floor(a * (1.0 / twopi)) * twopi;
  sincosf(float(a), s, c);
}

// store one element of the draft KV cache (fp32 or bf16 layout)
__device__ __forceinline__ void kv_store(void* base, size_t idx, float v, int f32) {
  if (f32) static_cast<float*>(base)[idx] = v;
  else static_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// ---- quantized draft KV (q8_0 K rows, q5_1 V rows; layout in kernels.hpp KvqRef) ----
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// byte offsets of row `pos` of KV head `head` in a region of nkv heads x cap rows
struct KvqAt {
  size_t k_code, k_scale, v_nib, v_hi, v_dm;
  __device__ KvqAt(int nkv, int cap, int hd, int head, int pos) {
    const size_t hr = (size_t)head * cap + pos, all = (size_t)nkv * cap;
    k_code = hr * hd;
    k_scale = all * hd + hr * (hd / 32) * 2;
    v_nib = hr * (hd / 2);
    v_hi = all * (hd / 2) + hr * (hd / 8);
    v_dm = all * (hd / 2 + hd / 8) + hr * (hd / 32) * 4;
  }
};

// q5_1 V code placement.  With NB = hd / 32 blocks, dim d = 32 b + 16 h + c (b < NB,
// h < 2, c < 16) keeps its low 4 bits in nibble h of byte B = c NB + b of the row's
// nibble array and its bit 4 in bit (B % 4) + 4 h of high-bit byte B / 4: the codes a
// lane c of an MFMA tile over dims 16 t + c needs are one contiguous run of bytes.
__device__ __forceinline__ int vq_byte(int dim, int hd) { return (dim & 15) * (hd >> 5) + (dim >> 5); }
__device__ __forceinline__ int vq_half(int dim) { return (dim >> 4) & 1; }
// the dim whose code sits in nibble h of byte B
__device__ __forceinline__ int vq_dim(int B, int h, int hd) {
  const int nb = hd >> 5, c = B / nb;
  return 32 * (B - c * nb) + 16 * h + c;
}

// Quantize one value per lane.  The lanes come in aligned groups of 32 holding dims
// [32b, 32b + 32) of one head row, K (q8_0) or V (q5_1); every lane of the wave calls
// it (the group reductions are shuffles); `on` lanes store.  K: the code and the
// block's scale are stored.  V: the block's (D, M) are stored and the 5-bit code is
// returned; kvq_pack_v writes a head row's codes once all of them are known.
// q8_0: D = fp16(max|x| / 127), q = clamp(rint(x / D), -127, 127), stored q + 128;
// q5_1: D = fp16((max - min) / 31), M = fp16(min), q = clamp(rint((x - M) / D), 0, 31);
// D == 0 gives code 0.  Subtraction and divisions are IEEE fp32.
__device__ __forceinline__ uint32_t kvq_quant(float x, bool is_k, int dim, uint8_t* kreg, uint8_t* vreg,
                                              const KvqAt& at, bool on) {
  float amax = fabsf(x), mn = x, mx = x;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  if (is_k) {
    const uint16_t Db = f32_to_f16_bits(__fdiv_rn(amax, 127.f));
    const float D = f16_bits_to_f32(Db);
    const float q = D > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(x, D)), -127.f), 127.f) : 0.f;
    if (on) {
      kreg[at.k_code + dim] = uint8_t(int(q) + 128);
      if ((dim & 31) == 0) *reinterpret_cast<uint16_t*>(kreg + at.k_scale + (dim >> 5) * 2) = Db;
    }
    return 0u;
  }
  const uint16_t Db = f32_to_f16_bits(__fdiv_rn(mx - mn, 31.f));
  const uint16_t Mb = f32_to_f16_bits(mn);
  const float D = f16_bits_to_f32(Db), M = f16_bits_to_f32(Mb);
  const float qf = D > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(x - M, D)), 0.f), 31.f) : 0.f;
  if (on && (dim & 31) == 0)
    *reinterpret_cast<uint32_t*>(vreg + at.v_dm + (dim >> 5) * 4) = uint32_t(Db) | (uint32_t(Mb) << 16);
  return uint32_t(qf);
}

// Write the nibble and high-bit bytes of one V head row from its 5-bit codes
// (codes[dim], dim < hd, e.g. in LDS); threads tid, tid + nthr, ... each write whole
// bytes.
__device__ __forceinline__ void kvq_pack_v(const uint8_t* codes, int hd, uint8_t* vreg, const KvqAt& at, int tid,
                                           int nthr) {
  for (int B = tid; B < hd / 2 + hd / 8; B += nthr) {
    if (B < hd / 2) {
      const uint32_t lo = codes[vq_dim(B, 0, hd)], hi = codes[vq_dim(B, 1, hd)];
      vreg[at.v_nib + B] = uint8_t((lo & 15u) | ((hi & 15u) << 4));
    } else {
      const int k = B - hd / 2;  // high bits of nibble bytes 4k .. 4k + 3
      uint32_t hb = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hb |= ((uint32_t(codes[vq_dim(4 * k + j, 0, hd)]) >> 4) & 1u) << j;
        hb |= ((uint32_t(codes[vq_dim(4 * k + j, 1, hd)]) >> 4) & 1u) << (j + 4);
      }
      vreg[at.v_hi + k] = uint8_t(hb);
    }
  }
}

}  // namespace e3
