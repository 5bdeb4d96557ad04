// Batched drafting: one decoder-layer step for up to 32 sequences at once.
//
// Every projection of the step is a skinny GEMM Y[b][r] = sum_k X[b][k] W[r][k]
// with b < 32, streamed once from HBM for all rows on the 32x32x16 bf16 MFMA:
// the activation rows are the A operand (staged through LDS in 512-wide k
// chunks), the weight rows the B operand, read straight from HBM into the
// fragment registers.  Inside a 64-wide k step a lane loads 64 contiguous bytes
// of its weight row and takes the matching activation slice from LDS: an MFMA
// sums over 16 k in any order, so both operands use the same permutation of k.
// Activations are (hi, lo) bf16 pairs and both halves are multiplied, which keeps
// ~16 mantissa bits of the fp32 activations.
//
// Around the GEMMs, one block per sequence row does what needs a whole row: the
// token and embedding gather, the RMSNorms, residual sums of split-K partials, the
// rotary embedding and the KV append, and the argmax over lm_head candidates.
#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBChunk = 512;           // k per LDS stage
constexpr int kBLdk = kBChunk + 8;     // padded LDS row (elements)
constexpr int kBVecPerChunk = 2 * kBatchRows * (kBChunk / 8);  // 16-byte vectors (hi and lo)

// Plain (cached) loads: a load instruction here touches 32 weight rows at 32
// bytes each and the next three instructions finish those lines; with the
// streaming hint the lines are not kept between them and the kernel fetches at
// about half the rate (measured on MI355X: lm_head 2.6 vs 5.0 TB/s).
__device__ __forceinline__ u32x4 ld_frag(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_bf16(float x, uint16_t* hi, uint16_t* lo) {
  const uint16_t h = f32_to_bf16(x);
  *hi = h;
  *lo = f32_to_bf16(x - bf16_to_f32(h));
}

// WM row tiles of 32 weight rows per block, WK waves per tile splitting each k chunk
template <int WM, int WK, int EPI>
__global__ __launch_bounds__(64 * WM * WK) void k_bgemm(const BGemmArgs a) {
  constexpr int NT = 64 * WM * WK;
  constexpr int KW = kBChunk / WK;   // k of one chunk per wave
  constexpr int STEPS = KW / 64;
  constexpr int VPT = kBVecPerChunk / NT;
  static_assert(KW % 64 == 0 && kBVecPerChunk % NT == 0, "chunk does not divide");
  static_assert(WM * (WK - 1) * 16 * 64 * 4 <= 2 * kBatchRows * kBLdk * 2, "reduction space");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * kBatchRows * kBLdk];
  __shared__ float sbv[WM][kBatchRows];
  __shared__ int sbi[WM][kBatchRows];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t = wv % WM, g = wv / WM;
  const int col = lane & 31, half = lane >> 5;
  const int row0 = blockIdx.x * (32 * WM) + t * 32;
  const uint16_t* wp = a.W + (size_t)min(row0 + col, a.N - 1) * a.K;
  const int k_begin = blockIdx.y * a.kb;
  const int k_end = min(a.K, k_begin + a.kb);

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;

  for (int c0 = k_begin; c0 < k_end; c0 += kBChunk) {
    // activation chunk (L2) first, then this wave's weight fragments (HBM)
    uint4 xv[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * NT;
      const int h = idx / (kBatchRows * 64);
      const int rem = idx - h * kBatchRows * 64;
      const int b = rem >> 6, k = c0 + (rem & 63) * 8;
      xv[i] = make_uint4(0, 0, 0, 0);
      if (b < a.m && k < k_end)
        xv[i] = *reinterpret_cast<const uint4*>((h ? a.Xlo : a.Xhi) + (size_t)b * a.ldx + k);
    }
    u32x4 w[STEPS][4];
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = c0 + g * KW + s * 64 + half * 32 + q * 8;
        w[s][q] = (u32x4){0u, 0u, 0u, 0u};
        if (k < k_end) w[s][q] = ld_frag(wp + k);
      }
    __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * NT;
      const int h = idx / (kBatchRows * 64);
      const int rem = idx - h * kBatchRows * 64;
      const int b = rem >> 6, kk = (rem & 63) * 8;
      *reinterpret_cast<uint4*>(&xs[(h * kBatchRows + b) * kBLdk + kk]) = xv[i];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (c0 + g * KW + s * 64 >= k_end) break;  // uniform over the wave
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = g * KW + s * 64 + half * 32 + q * 8;
        const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&xs[col * kBLdk + kk]);
        const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&xs[(kBatchRows + col) * kBLdk + kk]);
        const bf16x8 wb = __builtin_bit_cast(bf16x8, w[s][q]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, wb, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, wb, acc, 0, 0, 0);
      }
    }
  }

  // waves of one tile that split the chunks add up through LDS
  if constexpr (WK > 1) {
    __syncthreads();
    float* red = reinterpret_cast<float*>(xs);
    if (g > 0) {
#pragma unroll
      for (int v = 0; v < 16; ++v) red[(((g - 1) * WM + t) * 16 + v) * 64 + lane] = acc[v];
    }
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int gg = 1; gg < WK; ++gg)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] += red[(((gg - 1) * WM + t) * 16 + v) * 64 + lane];
    }
  }

  // D of a 32x32 tile: lane l holds weight row row0 + l % 32 for the batch rows
  // 8 * (v / 4) + 4 * (l / 32) + v % 4
  const int r = row0 + col;
  if constexpr (EPI == kBEpiPartial) {
    if (g == 0 && r < a.N) {
      float* P = a.P + (size_t)blockIdx.y * kBatchRows * a.N + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int b = 8 * (v >> 2) + 4 * half + (v & 3);
        if (b < a.m) P[(size_t)b * a.N] = acc[v];
      }
    }
  } else if constexpr (EPI == kBEpiSilu) {
    // rows 2i (gate) and 2i + 1 (up) sit in neighbouring lanes
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float other = __shfl_xor(acc[v], 1, kWave);
      const int b = 8 * (v >> 2) + 4 * half + (v & 3);
      if (g == 0 && !(col & 1) && r < a.N && b < a.m) {
        uint16_t hi, lo;
        split_bf16(silu(acc[v]) * other, &hi, &lo);
        const size_t o = (size_t)b * a.ld_act + (r >> 1);
        a.act_hi[o] = hi;
        a.act_lo[o] = lo;
      }
    }
  } else {
    // best (value, index) per batch row over this block's weight rows
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int b = 8 * (v >> 2) + 4 * half + (v & 3);
      float bv = r < a.N ? acc[v] : -INFINITY;
      int bi = r < a.N ? r : 0x7FFFFFFF;
      if (a.logits && g == 0 && r < a.N && b < a.m) a.logits[(size_t)b * a.N + r] = acc[v];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (g == 0 && col == 0) {
        sbv[t][b] = bv;
        sbi[t][b] = bi;
      }
    }
    __syncthreads();
    if (tid < a.m) {
      float bv = sbv[0][tid];
      int bi = sbi[0][tid];
#pragma unroll
      for (int tt = 1; tt < WM; ++tt)
        if (better(sbv[tt][tid], sbi[tt][tid], bv, bi)) { bv = sbv[tt][tid]; bi = sbi[tt][tid]; }
      a.cand_v[(size_t)tid * a.ncand + blockIdx.x] = bv;
      a.cand_i[(size_t)tid * a.ncand + blockIdx.x] = bi;
    }
  }
}

// launch shapes: (row tiles, waves per tile)
#define E3_BGEMM_VARIANTS(X) X(1, 2, 4) X(2, 1, 8)
constexpr int kBVariantRows[] = {128, 64, 32};

BGemmPlan bgemm_plan(int N, int K, int epi) {
  // a fused epilogue needs the whole K in one block
  BGemmPlan p{};
  const int chunks = (K + kBChunk - 1) / kBChunk;
  const int target = 768;  // blocks of the split-K form (three per CU)
  if (epi != kBEpiPartial) {
    p.variant = 1;
    const int rows = kBVariantRows[p.variant];
    if ((N + rows - 1) / rows < 256) p.variant = 2;
    p.splits = 1;
    p.kb = chunks * kBChunk;
  } else {
    p.variant = 1;
    const int rb = (N + kBVariantRows[1] - 1) / kBVariantRows[1];
    int sp = (target + rb - 1) / rb;
    if (sp > chunks) sp = chunks;
    if (sp < 1) sp = 1;
    const int per = (chunks + sp - 1) / sp;
    p.kb = per * kBChunk;
    p.splits = (K + p.kb - 1) / p.kb;
  }
  p.blocks = (N + kBVariantRows[p.variant] - 1) / kBVariantRows[p.variant];
  return p;
}

hipError_t launch_bgemm(BGemmArgs a, const BGemmPlan& p, int epi, hipStream_t s) {
  if (a.m < 1 || a.m > kBatchRows || (a.K & 7) || (a.ldx & 7)) return hipErrorInvalidValue;
  if (epi != kBEpiPartial && p.splits != 1) return hipErrorInvalidValue;
  if (epi == kBEpiArgmax && a.ncand < p.blocks) return hipErrorInvalidValue;
  a.kb = p.kb;
  dim3 grid(p.blocks, p.splits);
#define E3_BGEMM_CASE(V, WM, WK)                                                                 \
  if (p.variant == V) {                                                                          \
    if (epi == kBEpiPartial)                                                                     \
      hipLaunchKernelGGL((k_bgemm<WM, WK, kBEpiPartial>), grid, dim3(64 * WM * WK), 0, s, a);    \
    else if (epi == kBEpiSilu)                                                                   \
      hipLaunchKernelGGL((k_bgemm<WM, WK, kBEpiSilu>), grid, dim3(64 * WM * WK), 0, s, a);       \
    else                                                                                         \
      hipLaunchKernelGGL((k_bgemm<WM, WK, kBEpiArgmax>), grid, dim3(64 * WM * WK), 0, s, a);     \
    return hipGetLastError();                                                                    \
  }
  E3_BGEMM_VARIANTS(E3_BGEMM_CASE)
#undef E3_BGEMM_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// grid (rows, ceil(3n / 1024)): 4 consecutive values per thread
__global__ __launch_bounds__(256) void k_bpack_aux(const BatchRows br, const float* __restrict__ a0,
                                                   const float* __restrict__ a1,
                                                   const float* __restrict__ a2, int n,
                                                   uint16_t* __restrict__ Xhi,
                                                   uint16_t* __restrict__ Xlo, int ldx) {
  const int r = blockIdx.x;
  const int k = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (k >= 3 * n) return;
  const int seg = k / n, kk = k - seg * n;
  const float* a = seg == 0 ? a0 : (seg == 1 ? a1 : a2);
  const float4 v = *reinterpret_cast<const float4*>(a + (size_t)br.orig[r] * n + kk);
  const float x[4] = {v.x, v.y, v.z, v.w};
  uint16_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16(x[e], &h[e], &l[e]);
  *reinterpret_cast<uint2*>(Xhi + (size_t)r * ldx + k) =
      make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16));
  *reinterpret_cast<uint2*>(Xlo + (size_t)r * ldx + k) =
      make_uint2(uint32_t(l[0]) | (uint32_t(l[1]) << 16), uint32_t(l[2]) | (uint32_t(l[3]) << 16));
}

hipError_t launch_bpack_aux(const BatchRows& br, const float* a0, const float* a1, const float* a2,
                            int n, uint16_t* Xhi, uint16_t* Xlo, int ldx, hipStream_t s) {
  if (n & 3) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bpack_aux, dim3(br.m, (3 * n + 1023) / 1024), dim3(256), 0, s, br, a0, a1, a2,
                     n, Xhi, Xlo, ldx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One block per row; thread i holds the float4 groups i and i + kBRowThreads of it.
constexpr int kBRowVec = kBRowMax / 4 / kBRowThreads;

__device__ __forceinline__ void store_split4(uint16_t* hi, uint16_t* lo, float4 v) {
  const float x[4] = {v.x, v.y, v.z, v.w};
  uint16_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16(x[e], &h[e], &l[e]);
  *reinterpret_cast<uint2*>(hi) =
      make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16));
  *reinterpret_cast<uint2*>(lo) =
      make_uint2(uint32_t(l[0]) | (uint32_t(l[1]) << 16), uint32_t(l[2]) | (uint32_t(l[3]) << 16));
}

__device__ __forceinline__ float4 scale4(float4 v, float4 w, float s) {
  return make_float4(v.x * w.x * s, v.y * w.y * s, v.z * w.z * s, v.w * w.w * s);
}

__device__ __forceinline__ float sq4(float4 v) {
  return fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, v.w * v.w)));
}

__global__ __launch_bounds__(kBRowThreads) void k_bprep(const BPrepArgs a) {
  __shared__ float red[2 * (kBRowThreads / 64)];
  __shared__ float sv[kBRowThreads / 64];
  __shared__ int si[kBRowThreads / 64];
  __shared__ int s_tok;
  const int r = blockIdx.x, n = a.n, nv = n / 4;
  const int orig = a.br.orig[r];
  if (a.step == 0) {
    if (threadIdx.x == 0) s_tok = a.boundary_tok[orig];
  } else {
    const int i = block_argmax(a.cand_v + (size_t)r * a.ncand, a.cand_i + (size_t)r * a.ncand,
                               a.ncand, sv, si);
    if (threadIdx.x == 0) {
      if (i < 0 || i >= a.dv) atomicOr(a.status, kStatusNanLogits);  // every logit NaN
      const int ic = min(max(i, 0), a.dv - 1);
      const int t = ic + a.d2t[ic];
      a.out_ids[(size_t)orig * a.gamma + a.step - 1] = t;
      s_tok = t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && (s_tok < 0 || s_tok >= a.vocab)) atomicOr(a.status, kStatusBadToken);
  const int tok = min(max(s_tok, 0), a.vocab - 1);  // reads the nearest row
  const uint2* erow = reinterpret_cast<const uint2*>(a.embed + (size_t)tok * n);
  float4 ev[kBRowVec], gv[kBRowVec];
  float se = 0.f, sg = 0.f;
#pragma unroll
  for (int j = 0; j < kBRowVec; ++j) {
    const int v = threadIdx.x + j * kBRowThreads;
    ev[j] = gv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (v >= nv) continue;
    const uint2 ew = erow[v];
    ev[j] = make_float4(bf16_lo(ew.x), bf16_hi(ew.x), bf16_lo(ew.y), bf16_hi(ew.y));
    se += sq4(ev[j]);
    if (a.step == 0) {
      if (a.bnd) {
        gv[j] = reinterpret_cast<const float4*>(a.bnd + (size_t)a.br.slot[r] * n)[v];
      } else {
        for (int z = 0; z < a.S_enc; ++z) {
          const float4 p = reinterpret_cast<const float4*>(a.Penc + ((size_t)z * kBatchRows + r) * n)[v];
          gv[j].x += p.x; gv[j].y += p.y; gv[j].z += p.z; gv[j].w += p.w;
        }
      }
      reinterpret_cast<float4*>(a.G + (size_t)r * n)[v] = gv[j];
      if (a.dbg_hidden) reinterpret_cast<float4*>(a.dbg_hidden + (size_t)orig * (a.gamma + 1) * n)[v] = gv[j];
      sg += sq4(gv[j]);
    }
  }
  block_sum2(se, sg, red);
  const float ie = 1.0f / sqrtf(se / float(n) + a.eps);
  const float ig = 1.0f / sqrtf(sg / float(n) + a.eps);
  uint16_t* xh = a.Xhi + (size_t)r * a.ldx;
  uint16_t* xl = a.Xlo + (size_t)r * a.ldx;
#pragma unroll
  for (int j = 0; j < kBRowVec; ++j) {
    const int v = threadIdx.x + j * kBRowThreads;
    if (v >= nv) continue;
    store_split4(xh + 4 * v, xl + 4 * v, scale4(ev[j], reinterpret_cast<const float4*>(a.w_in)[v], ie));
    if (a.step == 0)
      store_split4(xh + n + 4 * v, xl + n + 4 * v,
                   scale4(gv[j], reinterpret_cast<const float4*>(a.w_hid)[v], ig));
  }
}

hipError_t launch_bprep(const BPrepArgs& a, hipStream_t s) {
  if ((a.n & 3) || a.n > kBRowMax || (a.ldx & 3)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bprep, dim3(a.m), dim3(kBRowThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// grid (rows, ceil(heads / 2)): two heads per block, one thread per pair of head rows
__global__ __launch_bounds__(128) void k_bqkv(const BQkvArgs a) {
  const int r = blockIdx.x, hd = a.head_dim;
  const int hs = blockIdx.y * 2 + threadIdx.x / 64;
  const int p = threadIdx.x % 64;
  if (hs >= a.n_head + 2 * a.n_head_kv) return;
  const int qd = a.n_head * hd;
  for (int pp = p; 2 * pp < hd; pp += 64) {
    const int row = hs * hd + 2 * pp;  // first of the pair in the (repacked) q|k|v rows
    float y0 = 0.f, y1 = 0.f;
    for (int z = 0; z < a.S; ++z) {
      const float2 v = *reinterpret_cast<const float2*>(a.P + ((size_t)z * kBatchRows + r) * a.N + row);
      y0 += v.x;
      y1 += v.y;
    }
    const int seg = hs < a.n_head ? 0 : (hs < a.n_head + a.n_head_kv ? 1 : 2);
    const int head = seg == 0 ? hs : (seg == 1 ? hs - a.n_head : hs - a.n_head - a.n_head_kv);
    const int pos = a.br.pos0[r] + a.step;
    const int li = 2 * pp;
    int d0 = li, d1 = li + 1;
    if (seg < 2 && li < a.rope_dim) {
      d0 = pp;
      d1 = pp + (a.rope_dim >> 1);
      float c, sn;
      rope_cs(pos, a.inv_freq[pp], &c, &sn);
      const float t0 = y0 * c - y1 * sn;
      const float t1 = y1 * c + y0 * sn;
      y0 = t0;
      y1 = t1;
    }
    if (seg == 0) {
      float* q = a.q + (size_t)r * qd + head * hd;
      q[d0] = y0;
      q[d1] = y1;
    } else {
      const size_t esz = a.kv_f32 ? 4 : 2;
      char* base = static_cast<char*>(a.kv) +
                   ((size_t)a.br.slot[r] * a.seq_elems + (seg == 2 ? a.seq_elems / 2 : 0)) * esz;
      const size_t at = ((size_t)head * a.cap + a.br.row0[r] + a.step) * hd;
      kv_store(base, at + d0, y0, a.kv_f32);
      kv_store(base, at + d1, y1, a.kv_f32);
    }
  }
}

hipError_t launch_bqkv(const BQkvArgs& a, hipStream_t s) {
  if (a.head_dim > 256 || (a.head_dim & 1) || (a.N & 1)) return hipErrorInvalidValue;
  const int heads = a.n_head + 2 * a.n_head_kv;
  hipLaunchKernelGGL(k_bqkv, dim3(a.m, (heads + 1) / 2), dim3(128), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBRowThreads) void k_bresid(const BResidArgs a) {
  __shared__ float red[2 * (kBRowThreads / 64)];
  const int r = blockIdx.x, n = a.n, nv = n / 4;
  float4 yv[kBRowVec];
  float ss = 0.f, dummy = 0.f;
  float* hid = a.dbg_hidden ? a.dbg_hidden + ((size_t)a.br.orig[r] * (a.gamma + 1) + a.step + 1) * n
                            : nullptr;
#pragma unroll
  for (int j = 0; j < kBRowVec; ++j) {
    const int v = threadIdx.x + j * kBRowThreads;
    yv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (v >= nv) continue;
    float4 y = reinterpret_cast<const float4*>(a.resid + (size_t)r * n)[v];
    for (int z = 0; z < a.S; ++z) {
      const float4 p = reinterpret_cast<const float4*>(a.P + ((size_t)z * kBatchRows + r) * n)[v];
      y.x += p.x; y.y += p.y; y.z += p.z; y.w += p.w;
    }
    yv[j] = y;
    reinterpret_cast<float4*>(a.y + (size_t)r * n)[v] = y;
    if (hid) reinterpret_cast<float4*>(hid)[v] = y;
    ss += sq4(y);
  }
  block_sum2(ss, dummy, red);
  const float inv = 1.0f / sqrtf(ss / float(n) + a.eps);
#pragma unroll
  for (int j = 0; j < kBRowVec; ++j) {
    const int v = threadIdx.x + j * kBRowThreads;
    if (v >= nv) continue;
    store_split4(a.x1_hi + (size_t)r * a.ld1 + 4 * v, a.x1_lo + (size_t)r * a.ld1 + 4 * v,
                 scale4(yv[j], reinterpret_cast<const float4*>(a.w1)[v], inv));
    if (a.x2_hi)
      store_split4(a.x2_hi + (size_t)r * a.ld2 + 4 * v, a.x2_lo + (size_t)r * a.ld2 + 4 * v,
                   scale4(yv[j], reinterpret_cast<const float4*>(a.w2)[v], inv));
  }
}

hipError_t launch_bresid(const BResidArgs& a, hipStream_t s) {
  if ((a.n & 3) || a.n > kBRowMax || (a.ld1 & 3) || (a.ld2 & 3)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bresid, dim3(a.m), dim3(kBRowThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bact(const float* __restrict__ P, int S, int n_ff,
                                              uint16_t* __restrict__ Xhi, uint16_t* __restrict__ Xlo,
                                              int ld) {
  const int r = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_ff) return;
  const size_t N = size_t(2) * n_ff;
  float gt = 0.f, up = 0.f;
  for (int z = 0; z < S; ++z) {
    const float2 v = *reinterpret_cast<const float2*>(P + ((size_t)z * kBatchRows + r) * N + 2 * i);
    gt += v.x;
    up += v.y;
  }
  split_bf16(silu(gt) * up, &Xhi[(size_t)r * ld + i], &Xlo[(size_t)r * ld + i]);
}

hipError_t launch_bact(const float* P, int S, int n_ff, int m, uint16_t* Xhi, uint16_t* Xlo, int ld,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_bact, dim3((n_ff + 255) / 256, m), dim3(256), 0, s, P, S, n_ff, Xhi, Xlo, ld);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// grid (bcand_count(N), m): a block sums the split-K partials of kBCandCols columns
// of one row, eight columns per thread, each split's loads in flight together
constexpr int kBCandPerThread = kBCandCols / 256;

__global__ __launch_bounds__(256) void k_bcand(const float* __restrict__ P, int S, int N,
                                               float* __restrict__ cand_v,
                                               int32_t* __restrict__ cand_i,
                                               float* __restrict__ logits) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int r = blockIdx.y, c0 = blockIdx.x * kBCandCols + threadIdx.x;
  float v[kBCandPerThread];
#pragma unroll
  for (int j = 0; j < kBCandPerThread; ++j) v[j] = 0.f;
  // two splits per round trip (the loads of both go out before either is added)
  int z = 0;
  for (; z + 1 < S; z += 2) {
    const float* p0 = P + ((size_t)z * kBatchRows + r) * N;
    const float* p1 = p0 + (size_t)kBatchRows * N;
    float a[kBCandPerThread], b[kBCandPerThread];
#pragma unroll
    for (int j = 0; j < kBCandPerThread; ++j) {
      const int c = c0 + 256 * j;
      a[j] = c < N ? p0[c] : 0.f;
      b[j] = c < N ? p1[c] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBCandPerThread; ++j) v[j] += a[j] + b[j];
  }
  if (z < S) {
    const float* pz = P + ((size_t)z * kBatchRows + r) * N;
#pragma unroll
    for (int j = 0; j < kBCandPerThread; ++j) {
      const int c = c0 + 256 * j;
      if (c < N) v[j] += pz[c];
    }
  }
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
#pragma unroll
  for (int j = 0; j < kBCandPerThread; ++j) {
    const int c = c0 + 256 * j;
    if (c < N) {
      if (logits) logits[(size_t)r * N + c] = v[j];
      if (better(v[j], c, bv, bi)) { bv = v[j]; bi = c; }
    }
  }
  wave_argmax(bv, bi);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k)
      if (better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
    const size_t at = (size_t)r * gridDim.x + blockIdx.x;
    cand_v[at] = bv;
    cand_i[at] = bi;
  }
}

hipError_t launch_bcand(const float* P, int S, int N, int m, float* cand_v, int32_t* cand_i,
                        float* logits, hipStream_t s) {
  if (m < 1 || m > kBatchRows || S < 1 || N < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bcand, dim3(bcand_count(N), m), dim3(256), 0, s, P, S, N, cand_v, cand_i,
                     logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bfinal(uint32_t* __restrict__ status, const BatchRows br, int gamma,
                                                const float* __restrict__ cand_v,
                                                const int32_t* __restrict__ cand_i, int ncand,
                                                const int32_t* __restrict__ d2t, int dv,
                                                int32_t* __restrict__ out_ids) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int r = blockIdx.x;
  const int i = block_argmax(cand_v + (size_t)r * ncand, cand_i + (size_t)r * ncand, ncand, sv, si);
  if (threadIdx.x == 0) {
    if (i < 0 || i >= dv) atomicOr(status, kStatusNanLogits);  // every logit NaN
    const int ic = min(max(i, 0), dv - 1);
    out_ids[(size_t)br.orig[r] * gamma + br.geff[r] - 1] = ic + d2t[ic];
  }
}

hipError_t launch_bfinal(uint32_t* status, const BatchRows& br, int m, int gamma, const float* cand_v,
                         const int32_t* cand_i, int ncand, const int32_t* d2t, int dv,
                         int32_t* out_ids, hipStream_t s) {
  hipLaunchKernelGGL(k_bfinal, dim3(m), dim3(256), 0, s, status, br, gamma, cand_v, cand_i, ncand, d2t, dv,
                     out_ids);
  return hipGetLastError();
}

}  // namespace e3
