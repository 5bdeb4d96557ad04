// Teacher-forced append of T rows (prefill and rebuild_after_verify):
//   A = [aux0 | aux1 | aux2] in 16-bit form  (pack)
//   F = A . W_fc^T                          (MFMA GEMM, fp32 out, optional split-K)
//   cat = 16-bit[RMSNorm(E[tok]) | RMSNorm(F)]
//   KV = cat . W_kv^T                       (MFMA GEMM over the k|v rows of W_qkv)
//   rotate k, store rows into the draft KV.
// The 16-bit forms: bf16 (hi, lo) pairs, so two products give fp32-grade rows; or
// one fp16 term against fp16 copies of the weights scaled by 2^8 (a bf16 weight
// times 2^8 is exact in fp16), 2^-8 applied when the products are summed.
// Only K and V of teacher-forced rows are ever read again, so Q, attention,
// the MLP and the head are not run for them.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace e3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// one 16x16x32 MFMA on 16-byte fragments holding bf16 or (F16) fp16 values
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(const bf16x8 a, const bf16x8 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp16 bits of x, raising kStatusAppendRange when x is outside the fp16 range
__device__ __forceinline__ uint16_t to_f16_checked(float x, uint32_t* status) {
  if (!(fabsf(x) < 65504.f)) atomicOr(status, kStatusAppendRange);
  return f32_to_f16_bits(x);
}

// dst[i] = fp16(src[i] * 2^8) for bf16 src: exact for 2^-25 <= |src| < 256 (eight
// significant bits fit an fp16 normal or a subnormal down to 2^-17); a weight the
// copy does not hold exactly raises kStatusAppendRange
__global__ __launch_bounds__(256) void k_bf16_to_f16_x256(const uint16_t* __restrict__ src,
                                                         uint16_t* __restrict__ dst, size_t count,
                                                         uint32_t* __restrict__ status) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float x = bf16_to_f32(src[i]) * 256.0f;
  const uint16_t h = f32_to_f16_bits(x);
  if (!(f16_bits_to_f32(h) == x)) atomicOr(status, kStatusAppendRange);
  dst[i] = h;
}

hipError_t launch_bf16_to_f16_x256(const uint16_t* src, uint16_t* dst, size_t count, uint32_t* status,
                                   hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bf16_to_f16_x256, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, src, dst,
                     count, status);
  return hipGetLastError();
}
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// grid (ceil(3n / 2048), T): 8 consecutive values per thread (they stay within one
// tap since n % 8 == 0), two 16-byte stores per plane
__global__ __launch_bounds__(256) void k_pack_aux(const float* __restrict__ a0,
                                                  const float* __restrict__ a1,
                                                  const float* __restrict__ a2, int T, int n,
                                                  uint16_t* __restrict__ A_hi,
                                                  uint16_t* __restrict__ A_lo, const TapRowsB yb,
                                                  int f16, uint32_t* __restrict__ status) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (t >= T || c >= 3 * n) return;
  const int j = c / n, k = c - j * n;
  const bool second = t >= yb.rows_x;  // rows from yb.rows_x on: the second set of streams
  const float* base = second ? (j == 0 ? yb.y[0] : (j == 1 ? yb.y[1] : yb.y[2]))
                             : (j == 0 ? a0 : (j == 1 ? a1 : a2));
  const float4* src = reinterpret_cast<const float4*>(base + (size_t)(second ? t - yb.rows_x : t) * n + k);
  const float4 v0 = src[0], v1 = src[1];
  const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint16_t h[8], l[8];
  if (f16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = to_f16_checked(v[e], status);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = f32_to_bf16(v[e]);
      l[e] = f32_to_bf16(v[e] - bf16_to_f32(h[e]));
    }
  }
  const size_t at = (size_t)t * 3 * n + c;
  *reinterpret_cast<uint4*>(A_hi + at) =
      make_uint4(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16),
                 uint32_t(h[4]) | (uint32_t(h[5]) << 16), uint32_t(h[6]) | (uint32_t(h[7]) << 16));
  if (A_lo)
    *reinterpret_cast<uint4*>(A_lo + at) =
        make_uint4(uint32_t(l[0]) | (uint32_t(l[1]) << 16), uint32_t(l[2]) | (uint32_t(l[3]) << 16),
                   uint32_t(l[4]) | (uint32_t(l[5]) << 16), uint32_t(l[6]) | (uint32_t(l[7]) << 16));
}

// ---------------------------------------------------------------------------
// The token table of the chain step's QKV embedding half (built at load):
// k_tok_ss: ss[t] = sum of E[t]^2 (one block per token row);
// k_pack_embed: rows [r0, r0 + T) of input_layernorm * E / rms(E) as bf16 (hi, lo)
// planes (rms from ss: sqrt(ss / n + eps)), the activations of the table GEMM, so the
// table holds the normalised embedding half.  grid (ceil(n / 2048), T), 8 values a
// thread.
__global__ __launch_bounds__(256) void k_tok_ss(const uint16_t* __restrict__ E, int n, float* __restrict__ ss) {
  __shared__ float red[8];
  const uint16_t* row = E + (size_t)blockIdx.x * n;
  float acc = 0.f;
  for (int c = threadIdx.x * 8; c < n; c += blockDim.x * 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + c);
    const float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                        bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(v[e], v[e], acc);
  }
  acc = wave_sum(acc);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) red[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) t += red[w];
    ss[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void k_pack_embed(const uint16_t* __restrict__ E, const float* __restrict__ w_in,
                                                    const float* __restrict__ ss, float eps, int r0, int T, int n,
                                                    uint16_t* __restrict__ A_hi, uint16_t* __restrict__ A_lo) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (t >= T || c >= n) return;
  const uint4 w = *reinterpret_cast<const uint4*>(E + (size_t)(r0 + t) * n + c);
  const float4 g0 = *reinterpret_cast<const float4*>(w_in + c), g1 = *reinterpret_cast<const float4*>(w_in + c + 4);
  const float ie = 1.0f / sqrtf(ss[r0 + t] / float(n) + eps);
  const float v[8] = {bf16_lo(w.x) * g0.x * ie, bf16_hi(w.x) * g0.y * ie, bf16_lo(w.y) * g0.z * ie,
                      bf16_hi(w.y) * g0.w * ie, bf16_lo(w.z) * g1.x * ie, bf16_hi(w.z) * g1.y * ie,
                      bf16_lo(w.w) * g1.z * ie, bf16_hi(w.w) * g1.w * ie};
  uint16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f32_to_bf16(v[e]);
    l[e] = f32_to_bf16(v[e] - bf16_to_f32(h[e]));
  }
  const size_t at = (size_t)t * n + c;
  *reinterpret_cast<uint4*>(A_hi + at) =
      make_uint4(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16),
                 uint32_t(h[4]) | (uint32_t(h[5]) << 16), uint32_t(h[6]) | (uint32_t(h[7]) << 16));
  *reinterpret_cast<uint4*>(A_lo + at) =
      make_uint4(uint32_t(l[0]) | (uint32_t(l[1]) << 16), uint32_t(l[2]) | (uint32_t(l[3]) << 16),
                 uint32_t(l[4]) | (uint32_t(l[5]) << 16), uint32_t(l[6]) | (uint32_t(l[7]) << 16));
}

hipError_t launch_tok_ss(const uint16_t* E, int vocab, int n, float* ss, hipStream_t s) {
  if (vocab <= 0 || (n & 7)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tok_ss, dim3(vocab), dim3(256), 0, s, E, n, ss);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_add_f32(float* __restrict__ dst, const float* __restrict__ src, size_t count) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    dst[i] += src[i];
}

hipError_t launch_add_f32(float* dst, const float* src, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((count + 255) / 256, 4096);
  hipLaunchKernelGGL(k_add_f32, dim3(unsigned(blocks)), dim3(256), 0, s, dst, src, count);
  return hipGetLastError();
}

hipError_t launch_pack_embed(const uint16_t* E, const float* w_in, const float* ss, float eps, int r0, int T, int n,
                             uint16_t* A_hi, uint16_t* A_lo, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if ((n & 7) || T > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_pack_embed, dim3((n + 2047) / 2048, T), dim3(256), 0, s, E, w_in, ss, eps, r0, T, n, A_hi,
                     A_lo);
  return hipGetLastError();
}

hipError_t launch_pack_aux(const float* a0, const float* a1, const float* a2, int T, int n,
                           uint16_t* A_hi, uint16_t* A_lo, hipStream_t s, const TapRowsB& yb, int f16,
                           uint32_t* status) {
  if (T <= 0) return hipSuccess;
  if ((n & 7) || T > 65535 || (f16 && A_lo)) return hipErrorInvalidValue;
  if (yb.rows_x < T && (!yb.y[0] || !yb.y[1] || !yb.y[2])) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_pack_aux, dim3((3 * n + 2047) / 2048, T), dim3(256), 0, s, a0, a1, a2, T, n,
                     A_hi, A_lo, yb, f16, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// sum of `splits` partials, loads issued four at a time
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int splits, size_t stride) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int z = 0;
  for (; z + 3 < splits; z += 4) {
    a0 += p[(size_t)z * stride];
    a1 += p[(size_t)(z + 1) * stride];
    a2 += p[(size_t)(z + 2) * stride];
    a3 += p[(size_t)(z + 3) * stride];
  }
  for (; z < splits; ++z) a0 += p[(size_t)z * stride];
  return (a0 + a1) + (a2 + a3);
}

__device__ __forceinline__ float4 sum_splits4(const float* __restrict__ p, int splits,
                                              size_t stride) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  int z = 0;
  for (; z + 1 < splits; z += 2) {
    const float4 u = *reinterpret_cast<const float4*>(p + (size_t)z * stride);
    const float4 v = *reinterpret_cast<const float4*>(p + (size_t)(z + 1) * stride);
    a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
    b.x += v.x; b.y += v.y; b.z += v.z; b.w += v.w;
  }
  if (z < splits) {
    const float4 u = *reinterpret_cast<const float4*>(p + (size_t)z * stride);
    a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
  }
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// One block per row: f = sum of the fc partials, the two RMSNorms, the concat.
__global__ __launch_bounds__(512) void k_tf_cat(uint32_t* __restrict__ status, const float* __restrict__ F,
                                                int splits,
                                                size_t f_split, int T, int n,
                                                const uint16_t* __restrict__ embed, int vocab,
                                                const int32_t* __restrict__ tok,
                                                const float* __restrict__ w_in,
                                                const float* __restrict__ w_hid, float eps,
                                                uint16_t* __restrict__ cat16,
                                                uint16_t* __restrict__ cat16_lo,
                                                float* __restrict__ cat32, const BndOut bnd,
                                                float f_scale, int f16) {
  extern __shared__ float fs[];  // [n]
  __shared__ float red[32];
  const int t = blockIdx.x;
  if (t >= T) {
    // a boundary row: f = sum of the partials, kept with f * w_hid and sum f^2 for the
    // next round's first step
    const int j = t - T;
    float* y = bnd.y + (size_t)bnd.slot[j] * n;
    float* yw = bnd.yw + (size_t)bnd.slot[j] * n;
    const float4* wh4 = reinterpret_cast<const float4*>(w_hid);
    float sf = 0.f, unused = 0.f;
    for (int i = threadIdx.x; i < (n >> 2); i += blockDim.x) {
      float4 f = sum_splits4(F + (size_t)t * n + 4 * i, splits, f_split);
      f = make_float4(f.x * f_scale, f.y * f_scale, f.z * f_scale, f.w * f_scale);
      const float4 wh = wh4[i];
      reinterpret_cast<float4*>(y)[i] = f;
      reinterpret_cast<float4*>(yw)[i] = make_float4(f.x * wh.x, f.y * wh.y, f.z * wh.z, f.w * wh.w);
      sf = fmaf(f.x, f.x, fmaf(f.y, f.y, fmaf(f.z, f.z, fmaf(f.w, f.w, sf))));
    }
    block_sum2(sf, unused, red);
    if (threadIdx.x == 0) bnd.ssq[bnd.slot[j]] = sf;
    return;
  }
  const int tid = tok[t];
  if (tid < 0 || tid >= vocab) {  // reads the nearest row, and says so
    if (threadIdx.x == 0) atomicOr(status, kStatusBadToken);
  }
  const int tk = min(max(tid, 0), vocab - 1);
  const uint2* e4 = reinterpret_cast<const uint2*>(embed + (size_t)tk * n);
  float4* f4 = reinterpret_cast<float4*>(fs);
  float se = 0.f, sf = 0.f;
  const int n4 = n >> 2;
#pragma unroll 2
  for (int i = threadIdx.x; i < n4; i += blockDim.x) {
    float4 f = sum_splits4(F + (size_t)t * n + 4 * i, splits, f_split);
    f = make_float4(f.x * f_scale, f.y * f_scale, f.z * f_scale, f.w * f_scale);
    f4[i] = f;
    sf = fmaf(f.x, f.x, fmaf(f.y, f.y, fmaf(f.z, f.z, fmaf(f.w, f.w, sf))));
    const uint2 u = e4[i];
    const float a0 = bf16_lo(u.x), a1 = bf16_hi(u.x), a2 = bf16_lo(u.y), a3 = bf16_hi(u.y);
    se = fmaf(a0, a0, fmaf(a1, a1, fmaf(a2, a2, fmaf(a3, a3, se))));
  }
  block_sum2(se, sf, red);
  const float ie = 1.0f / sqrtf(se / float(n) + eps);
  const float iff = 1.0f / sqrtf(sf / float(n) + eps);
  const float4* wi4 = reinterpret_cast<const float4*>(w_in);
  const float4* wh4 = reinterpret_cast<const float4*>(w_hid);
  for (int i = threadIdx.x; i < n4; i += blockDim.x) {
    const uint2 u = e4[i];
    const float4 wi = wi4[i], wh = wh4[i], f = f4[i];
    const float4 ea = make_float4(wi.x * (bf16_lo(u.x) * ie), wi.y * (bf16_hi(u.x) * ie),
                                  wi.z * (bf16_lo(u.y) * ie), wi.w * (bf16_hi(u.y) * ie));
    const float4 fb = make_float4(wh.x * (f.x * iff), wh.y * (f.y * iff), wh.z * (f.z * iff),
                                  wh.w * (f.w * iff));
    if (cat16) {
      uint16_t* row = cat16 + (size_t)t * 2 * n;
      const float cv[8] = {ea.x, ea.y, ea.z, ea.w, fb.x, fb.y, fb.z, fb.w};
      uint16_t h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = f16 ? to_f16_checked(cv[q], status) : f32_to_bf16(cv[q]);
      uint2 pa, pb;
      pa.x = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
      pa.y = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
      pb.x = uint32_t(h[4]) | (uint32_t(h[5]) << 16);
      pb.y = uint32_t(h[6]) | (uint32_t(h[7]) << 16);
      reinterpret_cast<uint2*>(row)[i] = pa;
      reinterpret_cast<uint2*>(row + n)[i] = pb;
      if (cat16_lo) {
        const float v[8] = {ea.x, ea.y, ea.z, ea.w, fb.x, fb.y, fb.z, fb.w};
        uint16_t l[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) l[q] = f32_to_bf16(v[q] - bf16_to_f32(h[q]));
        uint16_t* lrow = cat16_lo + (size_t)t * 2 * n;
        pa.x = uint32_t(l[0]) | (uint32_t(l[1]) << 16);
        pa.y = uint32_t(l[2]) | (uint32_t(l[3]) << 16);
        pb.x = uint32_t(l[4]) | (uint32_t(l[5]) << 16);
        pb.y = uint32_t(l[6]) | (uint32_t(l[7]) << 16);
        reinterpret_cast<uint2*>(lrow)[i] = pa;
        reinterpret_cast<uint2*>(lrow + n)[i] = pb;
      }
    } else {
      float* row = cat32 + (size_t)t * 2 * n;
      reinterpret_cast<float4*>(row)[i] = ea;
      reinterpret_cast<float4*>(row + n)[i] = fb;
    }
  }
}

hipError_t launch_tf_cat(uint32_t* status, const float* F, int splits, size_t f_split, int T, int n,
                         const uint16_t* embed, int vocab, const int32_t* tok, const float* w_in,
                         const float* w_hid, float eps, uint16_t* cat16, uint16_t* cat16_lo,
                         float* cat32, hipStream_t s, const BndOut* bnd, float f_scale, int f16) {
  if (f16 && (cat16_lo || !cat16)) return hipErrorInvalidValue;
  BndOut b{};
  if (bnd) {
    if (bnd->count < 0 || bnd->count > kBndRows || (bnd->count > 0 && (!bnd->y || !bnd->yw || !bnd->ssq)))
      return hipErrorInvalidValue;
    b = *bnd;
  }
  if (T < 0 || T + b.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_tf_cat, dim3(T + b.count), dim3(512), size_t(n) * sizeof(float), s, status, F, splits,
                     f_split, T, n, embed, vocab, tok, w_in, w_hid, eps, cat16, cat16_lo, cat32, b, f_scale,
                     f16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One block per row; a thread handles one adjacent (repacked) pair of k or v.
// One block per row; row t of the pass belongs to the segment s with
// row0[s] <= t < row0[s + 1], which is sequence slot[s] at position pos0[s] + (t - row0[s]).
__global__ __launch_bounds__(256) void k_tf_store(const float* __restrict__ P, int splits,
                                                  size_t p_split, const StoreSegs segs, int nkv,
                                                  int hd, int rope_dim,
                                                  const double* __restrict__ inv_freq,
                                                  char* __restrict__ kv, size_t seq_elems, int cap,
                                                  int kv_f32, float p_scale) {
  const int t = segs.row0[0] + blockIdx.x;
  int sg = 0;
  while (sg + 1 < segs.n && t >= segs.row0[sg + 1]) ++sg;
  const int kvd = nkv * hd;
  const int pos = segs.pos0[sg] + (t - segs.row0[sg]);
  const size_t esz = kv_f32 ? 4 : 2;
  char* k_cache = kv + (size_t)segs.slot[sg] * seq_elems * esz;
  char* v_cache = k_cache + seq_elems / 2 * esz;
  const float* row = P + (size_t)t * 2 * kvd;
  // grid.y spreads the kvd value pairs of a row over blocks (one pair per thread)
  for (int pr = blockIdx.y * blockDim.x + threadIdx.x; pr < kvd; pr += gridDim.y * blockDim.x) {
    const int r = 2 * pr;
    float y0 = sum_splits(row + r, splits, p_split) * p_scale;
    float y1 = sum_splits(row + r + 1, splits, p_split) * p_scale;
    const bool is_k = r < kvd;
    const int rr = is_k ? r : r - kvd;
    const int head = rr / hd, li = rr - head * hd;
    int d0 = li, d1 = li + 1;
    if (is_k && li < rope_dim) {
      const int i = li >> 1;
      d0 = i;
      d1 = i + (rope_dim >> 1);
      float c, sv;
      rope_cs(pos, inv_freq[i], &c, &sv);
      const float t0 = y0 * c - y1 * sv, t1 = y1 * c + y0 * sv;
      y0 = t0;
      y1 = t1;
    }
    void* base = is_k ? k_cache : v_cache;
    const size_t at = ((size_t)head * cap + pos) * hd;
    kv_store(base, at + d0, y0, kv_f32);
    kv_store(base, at + d1, y1, kv_f32);
  }
}

// k_tf_store for quantized regions: a block's 256 pairs are 512 consecutive values of
// the [k | v] row, i.e. whole heads (head_dim divides 512); they are rotated into
// LDS at their final dims, then quantized 32 dims at a time (one value per lane),
// and the V heads' codes packed into their nibble and high-bit bytes.
__global__ __launch_bounds__(256) void k_tf_store_q(const float* __restrict__ P, int splits,
                                                    size_t p_split, const StoreSegs segs, int nkv,
                                                    int hd, int rope_dim,
                                                    const double* __restrict__ inv_freq,
                                                    uint8_t* __restrict__ kv, size_t seq_bytes,
                                                    int cap, float p_scale) {
  __shared__ float srow[512];
  __shared__ uint8_t vcode[512];
  const int t = segs.row0[0] + blockIdx.x;
  int sg = 0;
  while (sg + 1 < segs.n && t >= segs.row0[sg + 1]) ++sg;
  const int kvd = nkv * hd;
  const int pos = segs.pos0[sg] + (t - segs.row0[sg]);
  uint8_t* kreg = kv + (size_t)segs.slot[sg] * seq_bytes;
  uint8_t* vreg = kreg + seq_bytes / 2;
  const float* row = P + (size_t)t * 2 * kvd;
  const int v0 = blockIdx.y * 512;  // this block's first value of the [k | v] row
  {
    const int r = v0 + 2 * threadIdx.x;
    if (r < 2 * kvd) {
      float y0 = sum_splits(row + r, splits, p_split) * p_scale;
      float y1 = sum_splits(row + r + 1, splits, p_split) * p_scale;
      const bool is_k = r < kvd;
      const int rr = is_k ? r : r - kvd;
      const int li = rr % hd;
      int d0 = li, d1 = li + 1;
      if (is_k && li < rope_dim) {
        const int i = li >> 1;
        d0 = i;
        d1 = i + (rope_dim >> 1);
        float c, sv;
        rope_cs(pos, inv_freq[i], &c, &sv);
        const float t0 = y0 * c - y1 * sv, t1 = y1 * c + y0 * sv;
        y0 = t0;
        y1 = t1;
      }
      const int hb = r - li - v0;  // the head's first value within the block
      srow[hb + d0] = y0;
      srow[hb + d1] = y1;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += blockDim.x) {  // two rounds, every lane
    const int v = v0 + i;
    const bool on = v < 2 * kvd;  // whole groups of 32 are on or off
    const bool is_k = v < kvd;
    const int rr = is_k ? v : v - kvd;
    const int head = rr / hd, dim = rr - head * hd;
    const KvqAt at(nkv, cap, hd, on ? head : 0, pos);
    vcode[i] = uint8_t(kvq_quant(on ? srow[i] : 0.f, is_k, dim, kreg, vreg, at, on));
  }
  __syncthreads();
  for (int h0 = 0; h0 < 512; h0 += hd) {  // the block's V heads (uniform)
    const int v = v0 + h0;
    if (v < kvd || v >= 2 * kvd) continue;
    const KvqAt at(nkv, cap, hd, (v - kvd) / hd, pos);
    kvq_pack_v(vcode + h0, hd, vreg, at, threadIdx.x, blockDim.x);
  }
}

hipError_t launch_tf_store(const float* P, int splits, size_t p_split, const StoreSegs& segs,
                           int n_head_kv, int head_dim, int rope_dim, const double* inv_freq, void* kv,
                           size_t seq_elems, int cap, int kv_f32, hipStream_t s, int kv_q, float p_scale) {
  if (segs.n < 1 || segs.n > kStoreSegs) return hipErrorInvalidValue;
  const int rows = segs.row0[segs.n] - segs.row0[0];
  if (rows <= 0) return hipSuccess;
  if (kv_q) {
    if (head_dim % 32 || 512 % head_dim) return hipErrorInvalidValue;
    const int blocks = (2 * n_head_kv * head_dim + 511) / 512;
    hipLaunchKernelGGL(k_tf_store_q, dim3(rows, blocks), dim3(256), 0, s, P, splits, p_split, segs,
                       n_head_kv, head_dim, rope_dim, inv_freq, static_cast<uint8_t*>(kv), seq_elems, cap,
                       p_scale);
    return hipGetLastError();
  }
  const int pair_blocks = (n_head_kv * head_dim + 255) / 256;
  hipLaunchKernelGGL(k_tf_store, dim3(rows, pair_blocks), dim3(256), 0, s, P, splits, p_split, segs, n_head_kv,
                     head_dim, rope_dim, inv_freq, static_cast<char*>(kv), seq_elems, cap, kv_f32, p_scale);
  return hipGetLastError();
}

// One thread per value: rows [row0, row0 + nrows) of quantized regions to fp32
// [row][nkv][hd] (K: D * (code - 128); V: fmaf(D, q, M)).
__global__ __launch_bounds__(256) void k_kvq_read(const uint8_t* __restrict__ kreg,
                                                  const uint8_t* __restrict__ vreg, int nkv, int cap,
                                                  int hd, int row0, int nrows, float* __restrict__ ko,
                                                  float* __restrict__ vo) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t per = (size_t)nkv * hd;
  if (i >= per * nrows) return;
  const int r = int(i / per), rem = int(i - (size_t)r * per);
  const int head = rem / hd, dim = rem - head * hd;
  const KvqAt at(nkv, cap, hd, head, row0 + r);
  const float Dk = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(kreg + at.k_scale + (dim >> 5) * 2));
  ko[i] = Dk * float(int(kreg[at.k_code + dim]) - 128);
  const int B = vq_byte(dim, hd), h = vq_half(dim);
  const uint32_t nb = vreg[at.v_nib + B];
  const uint32_t q = ((nb >> (4 * h)) & 15u) | (((uint32_t(vreg[at.v_hi + (B >> 2)]) >> ((B & 3) + 4 * h)) & 1u) << 4);
  const uint32_t dm = *reinterpret_cast<const uint32_t*>(vreg + at.v_dm + (dim >> 5) * 4);
  vo[i] = fmaf(f16_bits_to_f32(uint16_t(dm & 0xFFFFu)), float(q), f16_bits_to_f32(uint16_t(dm >> 16)));
}

hipError_t launch_kvq_read(const void* kreg, const void* vreg, int nkv, int cap, int hd, int row0,
                           int nrows, float* k_out, float* v_out, hipStream_t s) {
  const size_t total = (size_t)nkv * hd * nrows;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_kvq_read, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(kreg), static_cast<const uint8_t*>(vreg), nkv, cap, hd,
                     row0, nrows, k_out, v_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void k_gather_rows(uint16_t* __restrict__ dst, const uint16_t* __restrict__ src,
                              const int32_t* __restrict__ dst_rows,
                              const int32_t* __restrict__ src_rows, int row_len) {
  const uint16_t* s = src + (size_t)src_rows[blockIdx.x] * row_len;
  uint16_t* d = dst + (size_t)dst_rows[blockIdx.x] * row_len;
  for (int i = threadIdx.x; i < row_len; i += blockDim.x) d[i] = s[i];
}

hipError_t launch_gather_rows(uint16_t* dst, const uint16_t* src, const int32_t* dst_rows,
                              const int32_t* src_rows, int count, int row_len, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_rows, dim3(count), dim3(256), 0, s, dst, src, dst_rows, src_rows,
                     row_len);
  return hipGetLastError();
}

__global__ void k_bf16_to_f32(const uint16_t* __restrict__ src, float* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf16_to_f32(src[i]);
}

hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bf16_to_f32, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MFMA GEMM: C[z] = (A_hi + A_lo)[:, kz] . B[:, kz]^T, bf16 in, fp32 out.
// The weights B are exact in bf16; the activations may carry a bf16 remainder
// A_lo, which costs a second MFMA per fragment and gives fp32-grade products.
//
// C[z] = A[M, kz-range] . B[N, kz-range]^T on v_mfma_f32_16x16x32_bf16.
//
// Waves tile the block WM x WN, each owning (BM / WM) x (BN / WN) of C as 16 x 16
// MFMA tiles.  Operand tiles of BK columns go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane: a wave instruction fills 1 KB of LDS, lane
// l at byte 16 l), NST of them in a ring so the loads of tile t + NST - 1 are in
// flight while tile t is multiplied; one barrier per tile.  LDS rows are BK
// elements unpadded; chunk c (8 elements) of row r sits in slot c ^ swizzle(r),
// which keeps the 16-byte fragment reads free of bank conflicts.  With A_lo
// given, the (hi, lo) halves of A share every B fragment (two MFMAs).
// Block order: consecutive blocks go to different XCDs; every block of one XCD
// gets the same weight (N) tile range, so a weight tile is fetched into only one
// XCD's L2.
template <int BK>
__device__ __forceinline__ int tile_swizzle(int r) {
  return BK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define E3_WV(i) \
  case i:        \
    wait_vmcnt<i>(); \
    break;
    E3_WV(0) E3_WV(1) E3_WV(2) E3_WV(3) E3_WV(4) E3_WV(5) E3_WV(6) E3_WV(7) E3_WV(8) E3_WV(9)
    E3_WV(10) E3_WV(11) E3_WV(12) E3_WV(13) E3_WV(14) E3_WV(15) E3_WV(16) E3_WV(17) E3_WV(18)
    E3_WV(19) E3_WV(20) E3_WV(21) E3_WV(22) E3_WV(23) E3_WV(24) E3_WV(25) E3_WV(26) E3_WV(27)
    E3_WV(28) E3_WV(29) E3_WV(30) E3_WV(31) E3_WV(32) E3_WV(33) E3_WV(34) E3_WV(35) E3_WV(36)
    E3_WV(37) E3_WV(38) E3_WV(39) E3_WV(40) E3_WV(41) E3_WV(42) E3_WV(43) E3_WV(44) E3_WV(45)
    E3_WV(46) E3_WV(47) E3_WV(48) E3_WV(49) E3_WV(50) E3_WV(51) E3_WV(52) E3_WV(53) E3_WV(54)
    E3_WV(55) E3_WV(56) E3_WV(57) E3_WV(58) E3_WV(59) E3_WV(60) E3_WV(61) E3_WV(62) E3_WV(63)
#undef E3_WV
    default:  // beyond the counter's range: wait for everything
      wait_vmcnt<0>();
      break;
  }
}

template <int BM, int BN, int WM, int WN, bool SPLIT, int BK, int NST, bool F16 = false>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A2, int lda,
    const uint16_t* __restrict__ B, int ldb, float* __restrict__ C, int M, int N, int kper,
    int mt, int nt) {
  constexpr int TM = BM / (16 * WM), TN = BN / (16 * WN);
  static_assert(TM * 16 * WM == BM && TN * 16 * WN == BN, "waves must tile the block");
  constexpr int NW = WM * WN;
  constexpr int NSA = SPLIT ? 2 : 1;
  constexpr int CPR = BK / 8, RPI = 64 / CPR;  // chunks per row, rows per load instruction
  constexpr int IA = BM / RPI, IB = BN / RPI;
  static_assert(IA * RPI == BM && IB * RPI == BN, "rows per load instruction");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* As = smem;                        // [NST][NSA][BM * BK]
  uint16_t* Bs = smem + NST * NSA * BM * BK;  // [NST][BN * BK]

  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int n_t = xcd + 8 * (slot / mt), m_t = slot % mt;
  if (n_t >= nt) return;  // whole block idle (grid rounded up to the XCD pattern)
  const int m0 = m_t * BM, n0 = n_t * BN;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int kb = blockIdx.z * kper;
  float* Cz = C + (size_t)blockIdx.z * M * N;
  // load instructions this wave issues per tile (the count its vmcnt waits use)
  const int lpt = (IA / NW + (wv < IA % NW ? 1 : 0)) * NSA + IB / NW + (wv < IB % NW ? 1 : 0);

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

  const int lrow = lane / CPR, lslot = lane % CPR;
  auto issue = [&](int kt, int st) {
    for (int q = wv; q < IA; q += NW) {
      const int r = q * RPI + lrow;
      const size_t off = (size_t)min(m0 + r, M - 1) * lda + kt + 8 * (lslot ^ tile_swizzle<BK>(r));
#pragma unroll
      for (int h = 0; h < NSA; ++h)
        __builtin_amdgcn_global_load_lds(
            (const void*)((h ? A2 : A) + off),
            (void __attribute__((address_space(3)))*)(As + ((size_t)(st * NSA + h) * BM + q * RPI) * BK),
            16, 0, 0);
    }
    for (int q = wv; q < IB; q += NW) {
      const int r = q * RPI + lrow;
      __builtin_amdgcn_global_load_lds(
          (const void*)(B + (size_t)min(n0 + r, N - 1) * ldb + kt + 8 * (lslot ^ tile_swizzle<BK>(r))),
          (void __attribute__((address_space(3)))*)(Bs + ((size_t)st * BN + q * RPI) * BK), 16, 0, 0);
    }
  };

  const int ntiles = kper / BK;
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0)
    if (s0 < ntiles) issue(kb + s0 * BK, s0);
  for (int t = 0; t < ntiles; ++t) {
    const int st = t % NST;
    // tile t has landed once at most the later tiles' loads are outstanding
    if (t + NST - 2 < ntiles) wait_vmcnt_dyn((NST - 2) * lpt);
    else wait_vmcnt<0>();
    __syncthreads();  // every wave's part of tile t is in LDS; tile t - 1's stage is free
    if (t + NST - 1 < ntiles) issue(kb + (t + NST - 1) * BK, (t + NST - 1) % NST);
    const uint16_t* Ab = As + (size_t)st * NSA * BM * BK;
    const uint16_t* Bb = Bs + (size_t)st * BN * BK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      // 16x16x32 operands: lane l holds row l % 16, columns 8 (l / 16) .. + 7 of the step
      const int c = (kk >> 3) + (lane >> 4);
      bf16x8 bfr[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * 16 * TN + j * 16 + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bb[r * BK + 8 * (c ^ tile_swizzle<BK>(r))]);
      }
#pragma unroll
      for (int h = 0; h < NSA; ++h) {
        bf16x8 af[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = wm * 16 * TM + i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const bf16x8*>(&Ab[((size_t)h * BM + r) * BK + 8 * (c ^ tile_swizzle<BK>(r))]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = mfma16<F16>(af[i], bfr[j], acc[i][j]);
      }
    }
  }

  // D of a 16x16 tile: lane l holds column l % 16, rows 4 (l / 16) + v
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * 16 * TN + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 16 * TM + i * 16 + 4 * (lane >> 4) + v;
        if (row < M) Cz[(size_t)row * N + col] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------------------
// Skinny GEMM for M <= 32 activation rows (batched drafting, short appends):
// C[z][M][N] = (A_hi + A_lo)[M, kz-range] . B[N, kz-range]^T, B the weight stream.
// A block owns kSgRows weight rows.  Per 64-wide k step its 256 threads load the
// weight tile row-contiguously (eight lanes per 128-byte row slice) and the
// activation tile into registers kSgDepth steps ahead, then copy one step's
// registers into one of two LDS buffers right before that step's MFMAs: the
// registers keep kSgDepth x 24 KB per block in flight, several times what an LDS
// ring of the same footprint holds.  Waves tile the block 1 x 4, each owning
// 32 x 32 of C as 2 x 2 tiles of 16x16x32 MFMA.  One barrier per step: a buffer
// is rewritten two steps after its last read, and every wave has passed the
// barrier in between.  Refills past the last step re-read the last tile (in
// bounds, never used).  TILED: B is the step-tiled copy of the weights
// (launch_tile_weights: each block's [128 rows][64 k] step is one contiguous 16 KB
// run), which the DRAM pages serve far better than 128 bytes from each of 128 rows
// 8 KB or more apart (at M = 32: lm_head 55 -> 47 us, gate/up 47 -> 40, QKV 26 -> 22).
constexpr int kSgRows = 128;
constexpr int kSgBK = 64;
constexpr int kSgDepth = 4;  // even: a step's LDS buffer is its parity

// Epilogues (one split only, i.e. K whole): kBEpiSilu writes silu(gate) * up of the
// interleaved (gate, up) rows as (hi, lo) bf16; kBEpiArgmax writes, per activation
// row, the best (value, index) over the block's 128 weight rows (lowest index on
// ties) and optionally the logits.  kBEpiPartial stores C[z].
struct SgEpi {
  int m;              // activation rows written (<= M)
  uint16_t* act_hi;   // kBEpiSilu: [m][ld_act]
  uint16_t* act_lo;
  int ld_act;
  float* cand_v;      // kBEpiArgmax: [m][ncand], ncand >= gridDim.x
  int32_t* cand_i;
  int ncand;
  float* logits;      // kBEpiArgmax, optional: [m][N]
};

template <bool SPLIT, int EPI, bool F16 = false, bool TILED = false>
__global__ __launch_bounds__(256) void k_sgemm(const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ A2, int lda,
                                               const uint16_t* __restrict__ B, int ldb,
                                               float* __restrict__ C, int M, int N, int kper,
                                               int nt, SgEpi e) {
  constexpr int NSA = SPLIT ? 2 : 1;
  constexpr int D = kSgDepth;
  static_assert(D % 2 == 0, "buffer parity follows the ring slot");
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kSgRows * kSgBK];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NSA][32 * kSgBK];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // block b owns weight tile b (consecutive blocks, and so tiles, go to different XCDs)
  const int n_t = blockIdx.x;
  if (n_t >= nt) return;
  const int n0 = n_t * kSgRows;
  const int kb = blockIdx.z * kper;
  const int nsteps = kper / kSgBK;
  float* Cz = C + (size_t)blockIdx.z * M * N;

  // thread t loads weight rows (t >> 3) + 32 q and activation row t >> 3, chunk t & 7
  const int lr = tid >> 3, lc = tid & 7;
  const uint16_t* wp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (TILED)  // ldb = K: K / 64 step tiles per 128-row block
      wp[q] = B + ((size_t)n_t * (ldb / kSgBK) + kb / kSgBK) * (kSgRows * kSgBK) + (lr + 32 * q) * kSgBK + 8 * lc;
    else
      wp[q] = B + (size_t)min(n0 + lr + 32 * q, N - 1) * ldb + kb + 8 * lc;
  }
  constexpr size_t wstep = TILED ? size_t(kSgRows) * kSgBK : size_t(kSgBK);  // elements a step
  const size_t aoff = (size_t)min(lr, M - 1) * lda + kb + 8 * lc;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;
  // the ring: slot I holds one step's weight chunks and activation chunk(s); slots
  // are named statically (E3_SG_*(I) with a literal I) so they stay in registers
  u32x4 wreg[D][4], areg[D][NSA];  // native vectors: kept in registers
#define E3_SG_ISSUE(I, ST)                                                                   \
  {                                                                                          \
    const int st_ = min((ST), nsteps - 1), k_ = st_ * kSgBK;                                 \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) wreg[I][q] =                               \
        *reinterpret_cast<const u32x4*>(wp[q] + st_ * wstep);                                \
    _Pragma("unroll") for (int h = 0; h < NSA; ++h) areg[I][h] =                             \
        *reinterpret_cast<const u32x4*>((h ? A2 : A) + aoff + k_);                           \
  }
#define E3_SG_STEP(I, T)                                                                     \
  {                                                                                          \
    const int buf = (I) & 1;                                                                 \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                          \
      const int r = lr + 32 * q;                                                             \
      *reinterpret_cast<u32x4*>(&Ws[buf][r * kSgBK + 8 * (lc ^ tile_swizzle<kSgBK>(r))]) =   \
          wreg[I][q];                                                                        \
    }                                                                                        \
    _Pragma("unroll") for (int h = 0; h < NSA; ++h)                                          \
        *reinterpret_cast<u32x4*>(&As[buf][h][lr * kSgBK + 8 * (lc ^ tile_swizzle<kSgBK>(lr))]) = \
        areg[I][h];                                                                          \
    __syncthreads();                                                                         \
    E3_SG_ISSUE(I, (T) + D)                                                                  \
    _Pragma("unroll") for (int kk = 0; kk < kSgBK; kk += 32) {                               \
      const int c = (kk >> 3) + (lane >> 4);                                                 \
      bf16x8 bfr[2];                                                                         \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                        \
        const int r = wv * 32 + j * 16 + (lane & 15);                                        \
        bfr[j] = *reinterpret_cast<const bf16x8*>(                                           \
            &Ws[buf][r * kSgBK + 8 * (c ^ tile_swizzle<kSgBK>(r))]);                         \
      }                                                                                      \
      _Pragma("unroll") for (int h = 0; h < NSA; ++h) {                                      \
        bf16x8 af[2];                                                                        \
        _Pragma("unroll") for (int i2 = 0; i2 < 2; ++i2) {                                   \
          const int r = i2 * 16 + (lane & 15);                                               \
          af[i2] = *reinterpret_cast<const bf16x8*>(                                         \
              &As[buf][h][r * kSgBK + 8 * (c ^ tile_swizzle<kSgBK>(r))]);                    \
        }                                                                                    \
        _Pragma("unroll") for (int i2 = 0; i2 < 2; ++i2)                                     \
        _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i2][j] =                           \
            mfma16<F16>(af[i2], bfr[j], acc[i2][j]);                                         \
      }                                                                                      \
    }                                                                                        \
  }
  static_assert(kSgDepth == 4, "the ring below names four slots");
  E3_SG_ISSUE(0, 0)
  E3_SG_ISSUE(1, 1)
  E3_SG_ISSUE(2, 2)
  E3_SG_ISSUE(3, 3)
  int t0 = 0;
  for (; t0 + D <= nsteps; t0 += D) {
    E3_SG_STEP(0, t0)
    E3_SG_STEP(1, t0 + 1)
    E3_SG_STEP(2, t0 + 2)
    E3_SG_STEP(3, t0 + 3)
  }
  // the last, partial group of steps (uniform)
  if (t0 < nsteps) E3_SG_STEP(0, t0)
  if (t0 + 1 < nsteps) E3_SG_STEP(1, t0 + 1)
  if (t0 + 2 < nsteps) E3_SG_STEP(2, t0 + 2)
#undef E3_SG_STEP
#undef E3_SG_ISSUE

  // D of a 16x16 tile: lane l holds column l % 16, rows 4 (l / 16) + v
  if constexpr (EPI == kBEpiPartial) {
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wv * 32 + j * 16 + (lane & 15);
        if (col >= N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = i2 * 16 + 4 * (lane >> 4) + v;
          if (row < M) Cz[(size_t)row * N + col] = acc[i2][j][v];
        }
      }
  } else if constexpr (EPI == kBEpiSilu) {
    // gate row 2i and up row 2i + 1 sit in neighbouring lanes
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wv * 32 + j * 16 + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float up = __shfl_xor(acc[i2][j][v], 1, kWave);
          const int row = i2 * 16 + 4 * (lane >> 4) + v;
          if (!(col & 1) && col < N && row < e.m) {
            const float x = silu(acc[i2][j][v]) * up;
            const uint16_t hi = f32_to_bf16(x);
            const size_t o = (size_t)row * e.ld_act + (col >> 1);
            e.act_hi[o] = hi;
            e.act_lo[o] = f32_to_bf16(x - bf16_to_f32(hi));
          }
        }
      }
  } else {
    __shared__ float sbv[4][32];
    __shared__ int sbi[4][32];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i2 * 16 + 4 * (lane >> 4) + v;
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wv * 32 + j * 16 + (lane & 15);
          if (col < N) {
            if (e.logits && row < e.m) e.logits[(size_t)row * N + col] = acc[i2][j][v];
            if (better(acc[i2][j][v], col, bv, bi)) { bv = acc[i2][j][v]; bi = col; }
          }
        }
        // over the 16 lanes that share this row
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o, kWave);
          const int oi = __shfl_xor(bi, o, kWave);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if ((lane & 15) == 0) {
          sbv[wv][row] = bv;
          sbi[wv][row] = bi;
        }
      }
    __syncthreads();
    if (tid < e.m) {
      float bv = sbv[0][tid];
      int bi = sbi[0][tid];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (better(sbv[w][tid], sbi[w][tid], bv, bi)) { bv = sbv[w][tid]; bi = sbi[w][tid]; }
      e.cand_v[(size_t)tid * e.ncand + n_t] = bv;
      e.cand_i[(size_t)tid * e.ncand + n_t] = bi;
    }
  }
}

static hipError_t launch_sgemm(const uint16_t* A_hi, const uint16_t* A_lo, int lda, const uint16_t* B,
                               int ldb, float* C, int M, int N, int kper, int splits, hipStream_t s,
                               bool f16, bool tiled = false) {
  if (M > 32 || kper % kSgBK) return hipErrorInvalidValue;
  const int nt = (N + kSgRows - 1) / kSgRows;
  dim3 grid((nt + 7) / 8 * 8, 1, splits);
  const SgEpi e{};
  if (tiled) {
    if (f16 || !A_lo || ldb != kper * splits) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_sgemm<true, kBEpiPartial, false, true>), grid, dim3(256), 0, s, A_hi, A_lo, lda, B, ldb,
                       C, M, N, kper, nt, e);
  } else if (f16)
    hipLaunchKernelGGL((k_sgemm<false, kBEpiPartial, true>), grid, dim3(256), 0, s, A_hi, A_lo, lda, B, ldb, C,
                       M, N, kper, nt, e);
  else if (A_lo)
    hipLaunchKernelGGL((k_sgemm<true, kBEpiPartial>), grid, dim3(256), 0, s, A_hi, A_lo, lda, B, ldb, C,
                       M, N, kper, nt, e);
  else
    hipLaunchKernelGGL((k_sgemm<false, kBEpiPartial>), grid, dim3(256), 0, s, A_hi, A_lo, lda, B, ldb, C,
                       M, N, kper, nt, e);
  return hipGetLastError();
}

int sgemm_tiles(int N) { return (N + kSgRows - 1) / kSgRows; }

hipError_t launch_sgemm_fused(const BGemmArgs& a, int epi, hipStream_t s) {
  if (a.m < 1 || a.m > kBatchRows || a.K % kSgBK || (a.ldx & 7) || !a.Xlo) return hipErrorInvalidValue;
  const int nt = sgemm_tiles(a.N);
  SgEpi e{};
  e.m = a.m;
  e.act_hi = a.act_hi; e.act_lo = a.act_lo; e.ld_act = a.ld_act;
  e.cand_v = a.cand_v; e.cand_i = a.cand_i; e.ncand = a.ncand; e.logits = a.logits;
  dim3 grid((nt + 7) / 8 * 8, 1, 1);
  if (epi == kBEpiSilu) {
    if (a.N % 2) return hipErrorInvalidValue;
    if (a.tiled)
      hipLaunchKernelGGL((k_sgemm<true, kBEpiSilu, false, true>), grid, dim3(256), 0, s, a.Xhi, a.Xlo, a.ldx, a.W,
                         a.K, nullptr, kBatchRows, a.N, a.K, nt, e);
    else
      hipLaunchKernelGGL((k_sgemm<true, kBEpiSilu>), grid, dim3(256), 0, s, a.Xhi, a.Xlo, a.ldx, a.W, a.K,
                         nullptr, kBatchRows, a.N, a.K, nt, e);
  } else if (epi == kBEpiArgmax) {
    if (a.ncand < nt) return hipErrorInvalidValue;
    if (a.tiled)
      hipLaunchKernelGGL((k_sgemm<true, kBEpiArgmax, false, true>), grid, dim3(256), 0, s, a.Xhi, a.Xlo, a.ldx,
                         a.W, a.K, nullptr, kBatchRows, a.N, a.K, nt, e);
    else
      hipLaunchKernelGGL((k_sgemm<true, kBEpiArgmax>), grid, dim3(256), 0, s, a.Xhi, a.Xlo, a.ldx, a.W, a.K,
                         nullptr, kBatchRows, a.N, a.K, nt, e);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The step-tiled copy of a weight matrix W [N][K] (K % 64 == 0) for the skinny GEMM:
// T [ceil(N / 128)][K / 64][128][64], rows past N zero.  One thread per 16 bytes.
__global__ __launch_bounds__(256) void k_tile_weights(const uint16_t* __restrict__ W, int N, int K,
                                                      uint16_t* __restrict__ T, size_t chunks) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= chunks) return;
  const int kts = K / kSgBK;
  const int c = int(i % 8);
  const size_t t = i / 8;
  const int r = int(t % kSgRows);
  const size_t u = t / kSgRows;
  const int kt = int(u % kts);
  const size_t row = (u / kts) * kSgRows + r;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < size_t(N)) v = *reinterpret_cast<const uint4*>(W + row * size_t(K) + size_t(kt) * kSgBK + 8 * c);
  *reinterpret_cast<uint4*>(T + i * 8) = v;
}

size_t tiled_weight_elems(int N, int K) { return size_t((N + kSgRows - 1) / kSgRows) * kSgRows * size_t(K); }

hipError_t launch_tile_weights(const uint16_t* W, int N, int K, uint16_t* T, hipStream_t s) {
  if (N <= 0 || K <= 0 || K % kSgBK) return hipErrorInvalidValue;
  const size_t chunks = tiled_weight_elems(N, K) / 8;
  hipLaunchKernelGGL(k_tile_weights, dim3(unsigned((chunks + 255) / 256)), dim3(256), 0, s, W, N, K, T, chunks);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const uint16_t* A_hi, const uint16_t* A_lo, int lda, const uint16_t* Bt, float* C,
                             int M, int N, int K, const GemmPlan& plan, hipStream_t s) {
  const int splits = plan.splits;
  if (M <= 0 || M > 32 || N <= 0 || splits < 1 || K % (kSgBK * splits) || !A_lo || (lda & 7))
    return hipErrorInvalidValue;
  return launch_sgemm(A_hi, A_lo, lda, Bt, K, C, M, N, K / splits, splits, s, false, true);
}

// K tile: 32 with split activations (three stages fit), 64 otherwise (two stages)
constexpr int kBKSplit = 32, kBKPlain = 64;

// 256-row tiles once there are 256 rows (256 or 320 columns), 128 x 128 below, and
// the skinny GEMM up to 32 rows (batched drafting, short appends)
static int gemm_bm(int M) { return M >= 256 ? 256 : (M > 32 ? 128 : 32); }

GemmPlan gemm_plan(int M, int N, int K) {
  // Candidates: tile width bn and K split s (a power of two keeping whole 64-wide
  // K tiles).  The blocks run in ceil(tiles s / 256) rounds, each block doing
  // bn * K / s of work (per tile row), so the cost is rounds * bn / s; ties go
  // to the smaller s.  Every split adds an M x N fp32 partial to write and sum:
  // up to 4 splits for long appends, up to 16 for short ones (<= 256 rows), whose
  // few tiles would leave most CUs idle and whose partials are small next to the
  // weights they stream.  The 320-wide tile exists for widths that 256 tiles
  // cover in a count just past a multiple of 256 (5120 columns at 4096 rows: 320
  // tiles of 256, but 256 of 320, filling every CU once with no K split).
  const int bm = gemm_bm(M);
  const int max_sp = M <= 256 ? 16 : 4;
  if (bm == 32) {
    // the skinny GEMM (128 weight rows per block, up to three blocks per CU): the
    // smallest split giving about three blocks for every four CUs; more splits only
    // add partials (measured with cold weights at the 4096-wide shapes: lm_head and
    // gate/up 1, qkv 4, down and o_proj 8)
    const long long tiles = (N + kSgRows - 1) / kSgRows;
    GemmPlan p{kSgRows, 0};
    for (int sp = 1; sp <= max_sp; sp *= 2) {
      if (K % (kBKPlain * sp) != 0) continue;
      p.splits = sp;
      if (tiles * sp >= 192) break;
    }
    if (p.splits == 0) p.splits = 1;  // K not a multiple of 64: rejected at launch
    return p;
  }
  GemmPlan best{bm, 1};
  double best_cost = 1e30;
  // 256-row blocks come 320, 256 or 128 wide; a block's rate relative to the
  // 320-wide one (measured over full rounds at 4096 rows, fp16: 1169, 1088, 980
  // TFLOP/s) divides its cost, so a narrower tile wins only by filling more CUs
  // (the 1024-row K|V GEMM of the 4096-wide drafter: 128 x 2048 columns in 256 x 128
  // blocks split 4 ways, every CU once, 40 us against 56 us for 256 x 256 on half of them)
  const int widths[3] = {bm, 320, 128};
  const double rate[3] = {0.93, 1.0, 0.84};
  for (int w = 0; w < (bm == 256 ? 3 : 1); ++w) {
    const int bn = widths[w];
    const double eff = bm == 256 ? rate[w] : 1.0;
    const long long tiles = (long long)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    for (int sp = 1; sp <= max_sp; sp *= 2) {
      if (K % (kBKPlain * sp) != 0) continue;
      const double cost = double((tiles * sp + 255) / 256) * bn / sp / eff;
      if (cost < best_cost * (1 - 1e-9) || (cost < best_cost * (1 + 1e-9) && sp < best.splits)) {
        best_cost = cost;
        best = GemmPlan{bn, sp};
      }
    }
  }
  return best;
}

template <int BM, int BN, int WM, int WN, bool SPLIT, int BK, int NST, bool F16 = false>
static hipError_t launch_tiles(const uint16_t* A_hi, const uint16_t* A_lo, int lda,
                               const uint16_t* B, int ldb, float* C, int M, int N, int kper,
                               int splits, hipStream_t s) {
  constexpr int NSA = SPLIT ? 2 : 1;
  constexpr size_t lds = size_t(NST) * (NSA * BM + BN) * BK * 2;
  static_assert(lds <= 160 * 1024, "LDS ring exceeds a workgroup's LDS");
  static bool attr_set = false;  // the attribute is per kernel; setting it twice is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, SPLIT, BK, NST, F16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  const int nt8 = (nt + 7) / 8 * 8;
  dim3 grid(mt * nt8, 1, splits), block(WM * WN * 64);
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, SPLIT, BK, NST, F16>), grid, block, lds, s, A_hi, A_lo, lda, B,
                     ldb, C, M, N, kper, mt, nt);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* A_hi, const uint16_t* A_lo, int lda, const uint16_t* B,
                            int ldb, float* C, int M, int N, int K, const GemmPlan& plan,
                            hipStream_t s, bool f16) {
  const int splits = plan.splits;
  if (M <= 0 || N <= 0 || splits < 1 || K % (kBKPlain * splits) != 0 || (lda & 7) || (ldb & 7) ||
      (f16 && A_lo))
    return hipErrorInvalidValue;
  const int kper = K / splits;
  const int bm = gemm_bm(M);
  if (bm == 32) {
    if (plan.bn != kSgRows) return hipErrorInvalidValue;
    return launch_sgemm(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s, f16);
  }
  if (f16) {  // one fp16 product
    if (bm == 256 && plan.bn == 320)
      return launch_tiles<256, 320, 4, 4, false, kBKPlain, 2, true>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
    if (bm == 256 && plan.bn == 128)
      return launch_tiles<256, 128, 4, 4, false, kBKPlain, 2, true>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
    if (plan.bn != bm) return hipErrorInvalidValue;
    if (bm == 256)
      return launch_tiles<256, 256, 4, 4, false, kBKPlain, 2, true>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
    return launch_tiles<128, 128, 2, 2, false, kBKPlain, 3, true>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
  }
  if (bm == 256 && plan.bn == 320) {
    if (A_lo) return launch_tiles<256, 320, 4, 4, true, kBKSplit, 3>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
    return launch_tiles<256, 320, 4, 4, false, kBKPlain, 2>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
  }
  if (bm == 256 && plan.bn == 128) {
    if (A_lo) return launch_tiles<256, 128, 4, 4, true, kBKSplit, 3>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
    return launch_tiles<256, 128, 4, 4, false, kBKPlain, 2>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
  }
  if (plan.bn != bm) return hipErrorInvalidValue;
  if (A_lo) {
    if (bm == 256) return launch_tiles<256, 256, 4, 4, true, kBKSplit, 3>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
    return launch_tiles<128, 128, 2, 2, true, kBKSplit, 4>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
  }
  if (bm == 256) return launch_tiles<256, 256, 4, 4, false, kBKPlain, 2>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
  return launch_tiles<128, 128, 2, 2, false, kBKPlain, 3>(A_hi, A_lo, lda, B, ldb, C, M, N, kper, splits, s);
}

}  // namespace e3
