// Decode attention of one query row per head over the draft KV cache.
//
// Grid (S context splits, n_head_kv[, batch rows]).  A block owns `chunk`
// consecutive KV rows of one KV head and all G = n_head / n_head_kv query heads
// that read it (each K/V byte is fetched once per step).  A lane holds 8
// consecutive elements of a row (16 bytes of bf16 or 32 of fp32), so a row is
// spread over head_dim / 8 lanes and a wave covers 512 / head_dim rows per step;
// fewer lanes per row means fewer cross-lane steps per row for the dot products
// and the softmax bookkeeping, which bound this kernel rather than HBM.
// Single pass with an online softmax in base 2 (scores scaled by log2 e): each
// lane group keeps (m, l, o) per query head, m a reference within 2^8 of the
// running maximum; K and V of a row are requested together, several rows ahead.
// Lane groups and waves are merged with the log-sum-exp rule at the end.  With
// S > 1 each block stores (m, l, unnormalised o) and a second kernel combines the
// splits per query head; with S == 1 the block writes the normalised output.
#include "common.hpp"
#include "kernels.hpp"
#include "qkv_token.hpp"

#include <algorithm>
#include <cstdlib>
#include <mutex>

namespace e3 {

constexpr int kAttnWaves = 4;
constexpr int kAttnMaxChunk = 512;
constexpr int kAttnMfmaMaxChunk = 2048;  // the MFMA decode kernel's longest split
// 256 rather than 512: a 4096-row context over 4 KV heads then splits 64 ways, and its
// combine loads every split in one round trip (128 splits took two)
constexpr int kAttnSingleBlocks = 256;
constexpr int kAttnQmBlocks = 512;  // the q8q5 MFMA kernel's target (within attn_max_splits)

// 16 bytes of a KV row as floats: 8 bf16 or 4 fp32 values
template <typename KT>
struct KvVec;
template <>
struct KvVec<uint16_t> {
  static constexpr int E = 8;
  __device__ static void unpack(const uint4 w, float* v) {
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
};
template <>
struct KvVec<float> {
  static constexpr int E = 4;
  __device__ static void unpack(const uint4 w, float* v) {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
};

constexpr int kAttnLaneElems = 8;  // elements of a row per lane
constexpr float kRescale = 8.0f;   // log2 headroom of the online softmax reference

// ---------------------------------------------------------------------------
// Deferred QKV (AttnArgs dq): a draft step's q and new K/V row are finished in the
// attention kernel.  The previous kernel left hsum (the hidden half of every QKV row,
// divided by rms(g)); a block takes its KV head's rows of the repacked QKV matrix --
// the G query heads, then the K head and the V head, (G + 2) hd rows -- as rotary
// pairs (rows 2p, 2p + 1 of a head hold dims p and p + r/2 when 2p < r, dims 2p and
// 2p + 1 otherwise), adds the token table's row of the step's token (the embedding
// half, divided by rms(E[tok])), and rotates q and k at the step's position (the
// fused QKV kernel's epilogue).
constexpr int kDqPairs = 6;     // rotary pairs per thread, at most
constexpr int kDqThreads = 256;  // the attention blocks' size (kAttnWaves waves)
static_assert(kDqThreads == 64 * kAttnWaves, "the decode kernels' block size");

struct DqPre {
  ArgmaxBatch first;                 // the previous step's candidates (first batch)
  int tok0;                          // or the boundary token
  float h0[kDqPairs], h1[kDqPairs];  // normalised hidden-half sums of the thread's pairs
  double f[kDqPairs];                // their rotary frequencies (pairs that rotate)
};

// repacked QKV row of pair pp of KV head kvh's (G + 2) hd rows; hs = head slot (G: K,
// G + 1: V), p = pair within the head
__device__ __forceinline__ int dq_row(const AttnArgs& a, int kvh, int G, int pp, int* hs, int* p) {
  const int hd = a.head_dim, hp = hd >> 1;
  const int h = pp / hp;
  *hs = h;
  *p = pp - h * hp;
  const int qd = a.n_head * hd, kvd = a.n_head_kv * hd;
  const int base = h < G ? (kvh * G + h) * hd : (h == G ? qd + kvh * hd : qd + kvd + kvh * hd);
  return base + 2 * *p;
}

// The loads that do not depend on the token, issued before the block's K/V rows (a
// wave's loads complete in issue order, so the token's come first).  No loops and no
// blockDim (a load): the waits for these then leave the K/V loads in flight.
__device__ __forceinline__ void dq_issue(const AttnArgs& a, int kvh, int G, DqPre& pre) {
  pre.tok0 = qkv_token_load<kDqThreads>(a.dqa, pre.first);
  const int P = (G + 2) * (a.head_dim >> 1);
#pragma unroll
  for (int k = 0; k < kDqPairs; ++k) {
    const int pp = int(threadIdx.x) + k * kDqThreads;
    pre.h0[k] = 0.f;
    pre.h1[k] = 0.f;
    pre.f[k] = 0.0;
    if (pp < P) {
      int hs, p;
      const float2 h = *reinterpret_cast<const float2*>(a.dq_hsum + dq_row(a, kvh, G, pp, &hs, &p));
      pre.h0[k] = h.x;
      pre.h1[k] = h.y;
      if (hs <= G && 2 * p < a.dqa.rope_dim) pre.f[k] = a.dqa.inv_freq[p];
    }
  }
}

// Finish q (sq[g * HD + d], natural dims, unscaled) and the new row (snew[d] = K,
// snew[HD + d] = V, rounded as the cache stores them).  The owner block (its split
// holds row T - 1) stores the row to the cache and leaves the row's base-2 scores
// (score scale `scale`) in sdot[g]; sdot is read after the caller's next barrier.
// Every thread of the block (kDqThreads) calls it.
template <int HD>
__device__ __forceinline__ void dq_finish(const AttnArgs& a, int kvh, int G, int T, bool owner, const DqPre& pre,
                                          float scale, float* sq, float* snew, float* sdot, float* sv, int* si,
                                          int* st) {
  const QkvArgs& d = a.dqa;
  const int tok = qkv_token_from<false, kDqThreads>(d, pre.first, pre.tok0, sv, si, st);
  const int N = (a.n_head + 2 * a.n_head_kv) * HD;
  const float* trow = d.tok_tab + (size_t)tok * N;
  const int P = (G + 2) * (HD / 2);
  float t0[kDqPairs], t1[kDqPairs];
#pragma unroll
  for (int k = 0; k < kDqPairs; ++k) {
    const int pp = int(threadIdx.x) + k * kDqThreads;
    t0[k] = 0.f;
    t1[k] = 0.f;
    if (pp < P) {
      int hs, p;
      const float2 t = *reinterpret_cast<const float2*>(trow + dq_row(a, kvh, G, pp, &hs, &p));
      t0[k] = t.x;
      t1[k] = t.y;
    }
  }
#pragma unroll
  for (int k = 0; k < kDqPairs; ++k) {
    const int pp = int(threadIdx.x) + k * kDqThreads;
    if (pp >= P) break;
    int hs, p;
    (void)dq_row(a, kvh, G, pp, &hs, &p);
    float y0 = t0[k] + pre.h0[k];  // both halves arrive normalised
    float y1 = t1[k] + pre.h1[k];
    int d0 = 2 * p, d1 = 2 * p + 1;
    if (hs <= G && 2 * p < d.rope_dim) {
      d0 = p;
      d1 = p + (d.rope_dim >> 1);
      float c, s;
      rope_cs(d.pos, pre.f[k], &c, &s);
      const float r0 = y0 * c - y1 * s;
      const float r1 = y1 * c + y0 * s;
      y0 = r0;
      y1 = r1;
    }
    if (hs < G) {
      sq[hs * HD + d0] = y0;
      sq[hs * HD + d1] = y1;
    } else {
      if (!a.kv_f32) {  // the value a read of the bf16 cache gives
        y0 = bf16_to_f32(f32_to_bf16(y0));
        y1 = bf16_to_f32(f32_to_bf16(y1));
      }
      snew[(hs - G) * HD + d0] = y0;
      snew[(hs - G) * HD + d1] = y1;
    }
  }
  __syncthreads();
  if (!owner) return;
  const size_t row = ((size_t)kvh * a.cap + (T - 1)) * HD;
  for (int i = threadIdx.x; i < HD; i += kDqThreads) {
    kv_store(d.k_cache, row + i, snew[i], a.kv_f32);
    kv_store(d.v_cache, row + i, snew[HD + i], a.kv_f32);
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int g = wv; g < G; g += kDqThreads / 64) {
    float t = 0.f;
    for (int e = lane; e < HD; e += 64) t = fmaf(snew[e], sq[g * HD + e] * scale, t);
    t = wave_sum(t);
    if (lane == 0) sdot[g] = t;
  }
}

template <int HD, int G, typename KT, bool DQ = false>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a, int chunk, int S) {
  constexpr int E = KvVec<KT>::E;            // elements per 16-byte vector
  constexpr int NV = kAttnLaneElems / E;     // vectors per lane per row (K, and V)
  constexpr int LPR = HD / kAttnLaneElems;   // lanes per row
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * kAttnWaves;
  // rows in flight per lane group: three fp32 rows keep three waves per SIMD and
  // stream 32K-row contexts 6 % faster than two; four would leave two waves
  constexpr int kDepth = NV == 1 ? 4 : 3;
  static_assert(LPR <= 64 && RPW >= 1 && NV * E == kAttnLaneElems, "a row must fit in one wave");
  __shared__ float obuf[kAttnWaves][G][HD];
  __shared__ float s_M[kAttnWaves][G], s_L[kAttnWaves][G];
  // deferred QKV: the step's queries, its new K/V row and that row's scores
  __shared__ __align__(16) float dq_q[DQ ? G * HD : 1];
  __shared__ float dq_kv[DQ ? 2 * HD : 1], dq_s[DQ ? G : 1], dq_sv[DQ ? 16 : 1];
  __shared__ int dq_si[DQ ? 16 : 1], dq_st[DQ ? 16 : 1];

  const int s = blockIdx.x, kvh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  // element e of a lane's eight sits at dim(e): vector j = e / E of the lane is
  // elements [j * HD / NV + sub * E, + E), so one load instruction of vector j
  // reads a contiguous HD / NV stretch of each row (all of it when NV == 1)
  auto dim = [&](int e) { return (e / E) * (HD / NV) + sub * E + (e % E); };
  int T = a.T;
  size_t kv_off = 0;
  const float* qrow = a.q;
  float* part_o = a.part_o;
  float* part_ml = a.part_ml;
  if (a.batched) {
    const int rb = blockIdx.z;
    T = a.br.row0[rb] + a.step + 1;
    kv_off = (size_t)a.br.slot[rb] * a.seq_elems;
    qrow += (size_t)rb * a.n_head * HD;
    part_o += (size_t)rb * a.n_head * S * HD;
    part_ml += (size_t)rb * a.n_head * S * 2;
  }
  const int r0 = s * chunk;
  if (r0 >= T) return;  // a split past this row's context (batched rows are ragged)
  // deferred QKV: row T - 1 is made here, so the ring covers the rows before it and
  // the block whose split holds it takes it from LDS
  const bool owner = DQ && T - 1 < r0 + chunk;
  const int r1 = min(DQ ? T - 1 : T, r0 + chunk);
  const bool direct = S == 1 && !a.batched;
  // scores in base 2: s * log2(e) / sqrt(hd), so every exponential is one exp2
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  const KT* Kb = static_cast<const KT*>(a.k_cache) + kv_off + (size_t)kvh * a.cap * HD + sub * E;
  const KT* Vb = static_cast<const KT*>(a.v_cache) + kv_off + (size_t)kvh * a.cap * HD + sub * E;

  // ring of kDepth rows per lane group: slot i holds row rb + off + i * RPB and is
  // refilled with the row kDepth strides ahead once consumed.  Row indices are
  // clamped to r1 - 1, so every load is in bounds and unconditional; a slot that
  // holds a clamped row is never consumed.
  const int off = wv * RPW + slot;
  const int rlast = max(r1 - 1, 0);  // (an owner's ring may be empty: its loads are never consumed)
  DqPre pre;
  if constexpr (DQ) dq_issue(a, kvh, G, pre);
  uint4 kw[kDepth][NV], vw[kDepth][NV];
  auto load_row = [&](int i, int row) {
    row = min(row, rlast);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      kw[i][j] = *reinterpret_cast<const uint4*>(Kb + (size_t)row * HD + j * (HD / NV));
      vw[i][j] = *reinterpret_cast<const uint4*>(Vb + (size_t)row * HD + j * (HD / NV));
    }
  };
  int rb = r0;  // the block's current stride (uniform)
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load_row(i, rb + off + i * RPB);
  // q carries the score scale, so a row's dot product is its base-2 score
  if constexpr (DQ) dq_finish<HD>(a, kvh, G, T, owner, pre, scale, dq_q, dq_kv, dq_s, dq_sv, dq_si, dq_st);
  float qv[G][kAttnLaneElems];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e)
      qv[g][e] = (DQ ? dq_q[g * HD + dim(e)] : qrow[(size_t)(kvh * G + g) * HD + dim(e)]) * scale;
  float m[G], mr[G], l[G], acc[G][kAttnLaneElems];  // mr = m + kRescale
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    mr[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] = 0.f;
  }
  // consume ring slot i (its row valid), refill it with the row kDepth strides on
  auto step = [&](int i, int row) {
    float kf[kAttnLaneElems], vf[kAttnLaneElems];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      KvVec<KT>::unpack(kw[i][j], kf + j * E);
      KvVec<KT>::unpack(vw[i][j], vf + j * E);
    }
    load_row(i, row + kDepth * RPB);
    float d[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) t = fmaf(kf[e], qv[g][e], t);
      d[g] = t;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) d[g] = group_sum<LPR>(d[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // m is a reference at most kRescale below the running maximum, not the
      // maximum itself: (l, acc) are rescaled only when a score passes m by
      // more than kRescale, so weights stay below 2^kRescale.  The hardware
      // exp2 flushes results below 2^-126 to zero: such weights vanish next to
      // the row that set m (weight 1).
      const float sc = d[g];
      if (sc > mr[g]) {
        const float fo = __builtin_amdgcn_exp2f(m[g] - sc);  // 0 on the first row (m = -inf)
        l[g] *= fo;
#pragma unroll
        for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] *= fo;
        m[g] = sc;
        mr[g] = sc + kRescale;
      }
      const float p = __builtin_amdgcn_exp2f(sc - m[g]);
      l[g] += p;
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  };
  // strides in which every lane group's kDepth rows are valid: no per-row checks
  for (; rb + kDepth * RPB <= r1; rb += kDepth * RPB) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) step(i, rb + off + i * RPB);
  }
  // the last, partial stride
  if (rb < r1) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int rr = rb + off + i * RPB;
      if (rr >= r1) break;
      step(i, rr);
    }
  }

  // merge lane groups and waves: common maximum per head, then sums
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mw = wave_max(m[g]);
    if (lane == 0) s_M[wv][g] = mw;
  }
  __syncthreads();
  // the block's reference per head: the waves' and (owner) the new row's score
  auto block_ref = [&](int g) {
    float Mb = s_M[0][g];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, s_M[w][g]);
    if (DQ && owner) Mb = fmaxf(Mb, dq_s[g]);
    return Mb;
  };
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float Mb = block_ref(g);
    const float f = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - Mb);
    l[g] *= f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] *= f;
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] += __shfl_xor(l[g], o, kWave);
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] += __shfl_xor(acc[g][e], o, kWave);
    }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) obuf[wv][g][dim(e)] = acc[g][e];
      if (sub == 0) s_L[wv][g] = l[g];
    }
  }
  __syncthreads();

  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) {
    const int g = i / HD, dd = i - g * HD;
    float v = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      v += obuf[w][g][dd];
      L += s_L[w][g];
    }
    if (DQ && owner) {  // the new row, weight 2^(score - reference)
      const float fn = exp2f(dq_s[g] - block_ref(g));
      v = fmaf(fn, dq_kv[HD + dd], v);
      L += fn;
    }
    const int h = kvh * G + g;
    if (direct) a.out[(size_t)h * HD + dd] = v / L;
    else part_o[((size_t)h * S + s) * HD + dd] = v;
  }
  if (direct) return;
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    const float Mb = block_ref(g);
    float L = 0.f;
    for (int w = 0; w < kAttnWaves; ++w) L += s_L[w][g];
    if (DQ && owner) L += exp2f(dq_s[g] - Mb);
    const int h = kvh * G + g;
    part_ml[((size_t)h * S + s) * 2 + 0] = Mb;
    part_ml[((size_t)h * S + s) * 2 + 1] = L;
  }
}

// ---------------------------------------------------------------------------
// Verify-window attention (mid M): M query rows per head, query row m seeing cache
// rows 0..ctx+m (the window's own K/V are rows ctx..ctx+M-1).  The M * G query
// vectors of a KV head are taken GQ at a time by "query group" blocks that walk the
// same split of K/V rows as k_attn does for G heads, with a per-vector row limit.
// The blocks of one (KV head, split) tile are placed on one XCD (workgroups go to
// the XCDs round robin by linear id, so tile t's groups get ids t % 8 + 8 k), where
// they read the tile's rows through the same L2: the rows come from HBM about once
// for all M * G vectors.
template <int HD, int GQ, typename KT>
__global__ __launch_bounds__(256) void k_attn_mid(VerifyArgs a, int chunk, int S, int QG) {
  constexpr int E = KvVec<KT>::E;
  constexpr int NV = kAttnLaneElems / E;
  constexpr int LPR = HD / kAttnLaneElems;
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * kAttnWaves;
  constexpr int kDepth = NV == 1 ? 4 : 3;
  __shared__ float obuf[kAttnWaves][GQ][HD];
  __shared__ float s_M[kAttnWaves][GQ], s_L[kAttnWaves][GQ];

  const int nkv = a.n_head_kv, G = a.n_head / nkv;
  const int tiles = S * nkv;
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int tile = (slot / QG) * 8 + xcd, qg = slot % QG;
  if (tile >= tiles) return;
  const int s = tile % S, kvh = tile / S;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rs = lane / LPR, sub = lane % LPR;
  auto dim = [&](int e) { return (e / E) * (HD / NV) + sub * E + (e % E); };
  const int T = a.ctx + a.M;
  const int r0 = s * chunk, r1 = min(T, r0 + chunk);
  // this group's query vectors: j = qg * GQ + jj over (m, g), m-major
  int lim[GQ], qrow[GQ];
#pragma unroll
  for (int jj = 0; jj < GQ; ++jj) {
    const int j = qg * GQ + jj;
    const int m = j / G, g = j - m * G;
    const bool ok = m < a.M;
    lim[jj] = ok ? a.ctx + m : -1;                    // last row seen (inclusive)
    qrow[jj] = ok ? m * a.n_head + kvh * G + g : -1;  // (m, head) index
  }
  const bool direct = S == 1;
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  const KT* Kb = static_cast<const KT*>(a.k) + (size_t)kvh * a.cap * HD + sub * E;
  const KT* Vb = static_cast<const KT*>(a.v) + (size_t)kvh * a.cap * HD + sub * E;
  const int off = wv * RPW + rs;
  const int rlast = r1 - 1;
  uint4 kw[kDepth][NV], vw[kDepth][NV];
  auto load_row = [&](int i, int row) {
    row = min(row, rlast);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      kw[i][j] = *reinterpret_cast<const uint4*>(Kb + (size_t)row * HD + j * (HD / NV));
      vw[i][j] = *reinterpret_cast<const uint4*>(Vb + (size_t)row * HD + j * (HD / NV));
    }
  };
  int rb = r0;
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load_row(i, rb + off + i * RPB);
  float qv[GQ][kAttnLaneElems];
#pragma unroll
  for (int g = 0; g < GQ; ++g)
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e)
      qv[g][e] = qrow[g] >= 0 ? a.q[(size_t)qrow[g] * HD + dim(e)] * scale : 0.f;
  float m[GQ], mr[GQ], l[GQ], acc[GQ][kAttnLaneElems];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m[g] = -INFINITY;
    mr[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] = 0.f;
  }
  auto step = [&](int i, int row) {
    float kf[kAttnLaneElems], vf[kAttnLaneElems];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      KvVec<KT>::unpack(kw[i][j], kf + j * E);
      KvVec<KT>::unpack(vw[i][j], vf + j * E);
    }
    load_row(i, row + kDepth * RPB);
    float d[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) t = fmaf(kf[e], qv[g][e], t);
      d[g] = t;
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g) d[g] = group_sum<LPR>(d[g]);
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      if (row > lim[g]) continue;  // past this query row's window position
      const float sc = d[g];
      if (sc > mr[g]) {
        const float fo = __builtin_amdgcn_exp2f(m[g] - sc);
        l[g] *= fo;
#pragma unroll
        for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] *= fo;
        m[g] = sc;
        mr[g] = sc + kRescale;
      }
      const float p = __builtin_amdgcn_exp2f(sc - m[g]);
      l[g] += p;
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  };
  for (; rb + kDepth * RPB <= r1; rb += kDepth * RPB) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) step(i, rb + off + i * RPB);
  }
  if (rb < r1) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int rr = rb + off + i * RPB;
      if (rr >= r1) break;
      step(i, rr);
    }
  }
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const float mw = wave_max(m[g]);
    if (lane == 0) s_M[wv][g] = mw;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    float Mb = s_M[0][g];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, s_M[w][g]);
    const float f = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - Mb);
    l[g] *= f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] *= f;
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      l[g] += __shfl_xor(l[g], o, kWave);
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] += __shfl_xor(acc[g][e], o, kWave);
    }
  if (rs == 0) {
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) obuf[wv][g][dim(e)] = acc[g][e];
      if (sub == 0) s_L[wv][g] = l[g];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < GQ * HD; i += blockDim.x) {
    const int g = i / HD, dd = i - g * HD;
    if (qrow[g] < 0) continue;
    float v = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      v += obuf[w][g][dd];
      Ls += s_L[w][g];
    }
    if (direct) a.out[(size_t)qrow[g] * HD + dd] = v / Ls;
    else a.part_o[((size_t)qrow[g] * S + s) * HD + dd] = v;
  }
  if (direct) return;
  if (threadIdx.x < GQ && qrow[threadIdx.x] >= 0) {
    const int g = threadIdx.x;
    float Mb = s_M[0][g], Ls = 0.f;
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, s_M[w][g]);
    for (int w = 0; w < kAttnWaves; ++w) Ls += s_L[w][g];
    a.part_ml[((size_t)qrow[g] * S + s) * 2 + 0] = Mb;
    a.part_ml[((size_t)qrow[g] * S + s) * 2 + 1] = Ls;
  }
}

// ---------------------------------------------------------------------------
// Verify-window attention on MFMA.  A block takes 16 query vectors of one KV head
// (a query group) over one split of rows; each wave walks 32-row tiles of the split.
// Per tile, S^T = K Q^T as two 16x16 outputs of v_mfma_f32_16x16x32_bf16 (A = 16 K
// rows, B = the 16 query vectors; lane l holds row l % 16 and dims 8 (l / 16) .. + 7
// of a 32-wide k step, and gets S^T[rows 4 (l / 16) + v][query l % 16]).  A lane thus
// holds 8 scores of one query (rows 4g + v and 16 + 4g + v, g = l / 16): exactly an A
// operand of O += P V over the 32 rows, when the MFMA's k slot 8g + v stands for row
// 4g + v and slot 8g + 4 + v for row 16 + 4g + v; V's B operand is loaded in that
// row order, 16 bytes of a row per lane (the output tiles' dims interleaved to match).  O's D layout holds queries 4g + v, so the online
// softmax rescale factors move there by shuffles.  fp32 operands enter as bf16
// (hi, lo) pairs, x = hi + lo to 2^-18, and hi*hi + hi*lo + lo*hi is summed.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 fp32 -> bf16 (hi, lo), both rounded to nearest even (v_cvt_pk_bf16_f32):
// |x - hi - lo| <= 2^-18 |x|
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = (__bf16)x[i];
    lo[i] = (__bf16)(x[i] - (float)hi[i]);
  }
}

__device__ __forceinline__ float kv_elem(const float* p) { return *p; }
__device__ __forceinline__ float kv_elem(const uint16_t* p) { return bf16_to_f32(*p); }

template <int HD, typename KT>
__global__ __launch_bounds__(256) void k_attn_mid_mfma(VerifyArgs a, int chunk, int S, int QG) {
  constexpr int NT = HD / 16;  // 16-wide output dim tiles
  constexpr int KS = HD / 32;  // k steps of S
  constexpr bool F32 = sizeof(KT) == 4;
  // V elements per load (bf16: 16 bytes, or 8 at head_dim 64; fp32: one element,
  // which measured faster at 32K rows than 16-byte loads, 96.5 against 110.8 us)
  // and dims per group of output tiles
  constexpr int VE = F32 ? 1 : (KvVec<KT>::E < NT ? KvVec<KT>::E : NT);
  constexpr int VD = 16 * VE;
  __shared__ float so[kAttnWaves][16][HD + 4];
  __shared__ float sm[kAttnWaves][16], sl[kAttnWaves][16];

  const int nkv = a.n_head_kv, G = a.n_head / nkv;
  const int tiles = S * nkv;
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int tile = (slot / QG) * 8 + xcd, qg = slot % QG;
  if (tile >= tiles) return;
  const int s = tile % S, kvh = tile / S;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int T = a.ctx + a.M;
  const int r0 = s * chunk, r1 = min(T, r0 + chunk);
  // this lane's query (S layout): vector j = qg * 16 + c16 over (m, g), m-major
  const int jq = qg * 16 + c16, mq = jq / G;
  const bool qok = mq < a.M;
  const int lim = qok ? a.ctx + mq : -1;
  const int qrow = qok ? mq * a.n_head + kvh * G + (jq - mq * G) : -1;
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  bf16x8_t qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = qok ? a.q[(size_t)qrow * HD + 32 * ks + 8 * g4 + e] * scale : 0.f;
    split8(x, qh[ks], ql[ks]);
  }
  const KT* Kb = static_cast<const KT*>(a.k) + (size_t)kvh * a.cap * HD;
  const KT* Vb = static_cast<const KT*>(a.v) + (size_t)kvh * a.cap * HD;
  f32x4_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int rlast = r1 - 1;
  for (int tb = r0 + 32 * wv; tb < r1; tb += 32 * kAttnWaves) {
    // V's B operands (rows in slot order, dim 16 t + c16) are requested first, so
    // they arrive with K's
    // Output tile t = VE * grp + k holds dim VD * grp + VE * c16 + k (VE elements per
    // load, VD = 16 VE dims per group): one load per row and group gives a lane VE
    // tiles' operands, 16 lanes reading 16 VE contiguous elements.
    float vx[NT][8];
#pragma unroll
    for (int grp = 0; grp < HD / VD; ++grp)
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int row = min(tb + (v < 4 ? 4 * g4 + v : 16 + 4 * g4 + (v - 4)), rlast);
        const KT* vp = Vb + (size_t)row * HD + VD * grp + VE * c16;
        float e[8];
        if constexpr (VE == 1) {
          e[0] = kv_elem(vp);
        } else if constexpr (VE * sizeof(KT) == 16) {
          KvVec<KT>::unpack(*reinterpret_cast<const uint4*>(vp), e);
        } else {  // 4 bf16
          const uint2 w = *reinterpret_cast<const uint2*>(vp);
          e[0] = bf16_lo(w.x); e[1] = bf16_hi(w.x); e[2] = bf16_lo(w.y); e[3] = bf16_hi(w.y);
        }
#pragma unroll
        for (int k = 0; k < VE; ++k) vx[VE * grp + k][v] = e[k];
      }
    // S^T for rows tb + 16 h + (0..15): A = K rows, B = queries
    f32x4_t st[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const KT* kr = Kb + (size_t)min(tb + 16 * h + c16, rlast) * HD + 8 * g4;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (F32) {
          const float4 u = *reinterpret_cast<const float4*>(kr + 32 * ks);
          const float4 w = *reinterpret_cast<const float4*>(kr + 32 * ks + 4);
          const float x[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
          bf16x8_t kh, kl;
          split8(x, kh, kl);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[ks], acc, 0, 0, 0);
        } else {
          const bf16x8_t kh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + 32 * ks));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], acc, 0, 0, 0);
        }
      }
      st[h] = acc;
    }
    // mask, tile maximum and sum per query (the 4 lanes c16, c16 + 16, ...)
    float sc[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ra = tb + 4 * g4 + v, rb = tb + 16 + 4 * g4 + v;
      sc[v] = (ra < r1 && ra <= lim) ? st[0][v] : -INFINITY;
      sc[4 + v] = (rb < r1 && rb <= lim) ? st[1][v] : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 8; ++v) mx = fmaxf(mx, sc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mn = fmaxf(m, mx);
    const float fo = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);  // m = -inf: 0
    float p[8], ps = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      p[v] = sc[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[v] - mn);
      ps += p[v];
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l = l * fo + ps;
    m = mn;
    // rescale O (D layout: queries 4 g4 + v) by those queries' factors
    float fv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) fv[v] = __shfl(fo, 4 * g4 + v, kWave);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[t][v] *= fv[v];
    bf16x8_t ph, pl;
    split8(p, ph, pl);
    // O += P V: B = V[rows (slot order)][dim 16 t + c16]
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float (&x)[8] = vx[t];
      if constexpr (F32) {
        bf16x8_t vh, vl;
        split8(x, vh, vl);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vh, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vl, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vh, o[t], 0, 0, 0);
      } else {
        bf16x8_t vh, vl;
        split8(x, vh, vl);  // exact: lo is zero for bf16 values
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vh, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vh, o[t], 0, 0, 0);
      }
    }
  }
  // merge the waves
  if (g4 == 0) {
    sm[wv][c16] = m;
    sl[wv][c16] = l;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) so[wv][4 * g4 + v][VD * (t / VE) + VE * c16 + (t % VE)] = o[t][v];
  __syncthreads();
  const bool direct = S == 1;
  for (int i = threadIdx.x; i < 16 * HD; i += blockDim.x) {
    const int q = i / HD, dd = i - q * HD;
    const int j = qg * 16 + q, mm = j / G;
    if (mm >= a.M) continue;
    const int qr = mm * a.n_head + kvh * G + (j - mm * G);
    float Mb = sm[0][q];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, sm[w][q]);
    float v = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = (Mb == -INFINITY || sm[w][q] == -INFINITY) ? 0.f : exp2f(sm[w][q] - Mb);
      v = fmaf(f, so[w][q][dd], v);
      Ls = fmaf(f, sl[w][q], Ls);
    }
    if (direct) a.out[(size_t)qr * HD + dd] = v / Ls;
    else {
      a.part_o[((size_t)qr * S + s) * HD + dd] = v;
      if (dd == 0) {
        a.part_ml[((size_t)qr * S + s) * 2 + 0] = Mb;
        a.part_ml[((size_t)qr * S + s) * 2 + 1] = Ls;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode attention over bf16 K/V on MFMA (head_dim 64 or 128, up to 16 query heads
// per KV head).  Same grid, partials and batched form as k_attn.  The G query
// vectors of the block's KV head are the 16 columns of an MFMA operand (unused
// columns zero): per 16-row tile, S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (A = 16
// K rows straight from memory, exact in bf16; B = the queries as bf16 (hi, lo)
// pairs, two products), which leaves lane (query c16, group g4) holding the scores
// of rows 4 g4 + v -- exactly the A operand of O += P V on v_mfma_f32_16x16x16bf16_1k
// (rows = queries, k = the tile's rows), P entering as (hi, lo) pairs against exact
// bf16 V.  V's B operand holds dim 16-column c16 over rows 4 g4 + v; a lane loads
// 16 bytes (8 dims) of each of its 4 rows, so output tile k holds dims 8 c16 + k.
// Tiles of a block go to its 4 waves round robin; each wave keeps the next
// kMfmaRing tiles' loads in flight while it computes.  The online softmax keeps a
// reference maximum per query that moves only when a tile's maximum passes it by
// more than kRescale (weights stay below 2^kRescale), so O is rarely rescaled.
typedef short bf16x4s_t __attribute__((ext_vector_type(4)));
constexpr int kMfmaRing = 2;

template <int HD, bool DQ = false>
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a, int chunk, int S) {
  constexpr int NT = HD / 16;               // output tiles of 16 dims
  constexpr int KS = HD / 32;               // k steps of S
  constexpr int VE = 8 < NT ? 8 : NT;       // bf16 elements per V load
  constexpr int VD = 16 * VE;               // dims per group of output tiles
  constexpr int NG = HD / VD;
  constexpr int R = kMfmaRing;
  constexpr int STRIDE = 16 * kAttnWaves;   // rows between a wave's consecutive tiles
  static_assert(NT * 16 == HD && KS * 32 == HD && NG * VD == HD, "head_dim 64 or 128");
  __shared__ float so[kAttnWaves][16][HD + 4];
  __shared__ float sm[kAttnWaves][16], sl[kAttnWaves][16];
  // deferred QKV: the step's queries, its new K/V row and that row's scores
  __shared__ __align__(16) float dq_q[DQ ? 16 * HD : 1];
  __shared__ float dq_kv[DQ ? 2 * HD : 1], dq_s[DQ ? 16 : 1], dq_sv[DQ ? 16 : 1];
  __shared__ int dq_si[DQ ? 16 : 1], dq_st[DQ ? 16 : 1];

  const int s = blockIdx.x, kvh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int G = a.n_head / a.n_head_kv;
  int T = a.T;
  size_t kv_off = 0;
  const float* qrow = a.q;
  float* part_o = a.part_o;
  float* part_ml = a.part_ml;
  if (a.batched) {
    const int rb = blockIdx.z;
    T = a.br.row0[rb] + a.step + 1;
    kv_off = (size_t)a.br.slot[rb] * a.seq_elems;
    qrow += (size_t)rb * a.n_head * HD;
    part_o += (size_t)rb * a.n_head * S * HD;
    part_ml += (size_t)rb * a.n_head * S * 2;
  }
  const int r0 = s * chunk;
  if (r0 >= T) return;  // a split past this row's context (batched rows are ragged)
  // deferred QKV: row T - 1 is made here, so the tiles cover the rows before it and
  // the block whose split holds it takes it from LDS
  const bool owner = DQ && T - 1 < r0 + chunk;
  const int r1 = min(DQ ? T - 1 : T, r0 + chunk);
  const bool direct = S == 1 && !a.batched;
  const int rlast = max(r1 - 1, 0);
  DqPre pre;
  if constexpr (DQ) dq_issue(a, kvh, G, pre);
  const uint16_t* Kb = static_cast<const uint16_t*>(a.k_cache) + kv_off + (size_t)kvh * a.cap * HD;
  const uint16_t* Vb = static_cast<const uint16_t*>(a.v_cache) + kv_off + (size_t)kvh * a.cap * HD;

  // ring slot i: K rows tb + c16 (dims 32 ks + 8 g4 ..), V rows tb + 4 g4 + v (dims
  // VD grp + VE c16 ..); row indices clamped to r1 - 1, masked when scored
  uint4 kr[R][KS];
  uint4 vr[R][NG][4];
  auto load = [&](int i, int tb) {
    const uint16_t* kp = Kb + (size_t)min(tb + c16, rlast) * HD + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[i][ks] = *reinterpret_cast<const uint4*>(kp + 32 * ks);
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint16_t* vp = Vb + (size_t)min(tb + 4 * g4 + v, rlast) * HD + VD * grp + VE * c16;
        if constexpr (VE == 8) {
          vr[i][grp][v] = *reinterpret_cast<const uint4*>(vp);
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(vp);
          vr[i][grp][v] = make_uint4(w.x, w.y, 0u, 0u);
        }
      }
  };
  const int tb0 = r0 + 16 * wv;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (tb0 + i * STRIDE < r1) load(i, tb0 + i * STRIDE);

  // queries carry the base-2 score scale; columns past G are zero
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  if constexpr (DQ) dq_finish<HD>(a, kvh, G, T, owner, pre, scale, dq_q, dq_kv, dq_s, dq_sv, dq_si, dq_st);
  const bool qok = c16 < G;
  bf16x8_t qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float* qp = DQ ? dq_q + (qok ? c16 : 0) * HD + 32 * ks + 8 * g4
                         : qrow + (size_t)(kvh * G + (qok ? c16 : 0)) * HD + 32 * ks + 8 * g4;
    const float4 u = *reinterpret_cast<const float4*>(qp), w = *reinterpret_cast<const float4*>(qp + 4);
    float x[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = qok ? x[e] * scale : 0.f;
    split8(x, qh[ks], ql[ks]);
  }
  f32x4_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  auto step = [&](int i, int tb) {
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t kh = __builtin_bit_cast(bf16x8_t, kr[i][ks]);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], st, 0, 0, 0);
    }
    uint4 vv[NG][4];
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
      for (int v = 0; v < 4; ++v) vv[grp][v] = vr[i][grp][v];
    if (tb + R * STRIDE < r1) load(i, tb + R * STRIDE);
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = (tb + 4 * g4 + v < r1) ? st[v] : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float fo = 1.f;
    if (mx > m + kRescale) {
      fo = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
      m = mx;
    }
    float pr[4], ps = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pr[v] = sc[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[v] - m);
      ps += pr[v];
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l = l * fo + ps;
    if (__any(fo != 1.f)) {  // O's D layout holds queries 4 g4 + v
      float fv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) fv[v] = __shfl(fo, 4 * g4 + v, kWave);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[t][v] *= fv[v];
    }
    bf16x4s_t ph, pl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const __bf16 h = (__bf16)pr[v];
      ph[v] = __builtin_bit_cast(short, h);
      pl[v] = __builtin_bit_cast(short, (__bf16)(pr[v] - (float)h));
    }
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
      for (int k = 0; k < VE; ++k) {
        bf16x4s_t vk;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 w = vv[grp][v];
          const uint32_t word = k < 2 ? w.x : k < 4 ? w.y : k < 6 ? w.z : w.w;
          vk[v] = (k & 1) ? short(word >> 16) : short(word & 0xffffu);
        }
        const int t = VE * grp + k;
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vk, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vk, o[t], 0, 0, 0);
      }
  };
  int tb = tb0;
  for (; tb + (R - 1) * STRIDE < r1; tb += R * STRIDE) {
#pragma unroll
    for (int i = 0; i < R; ++i) step(i, tb + i * STRIDE);
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (tb + i * STRIDE < r1) step(i, tb + i * STRIDE);

  // merge the waves
  if (g4 == 0) {
    sm[wv][c16] = m;
    sl[wv][c16] = l;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) so[wv][4 * g4 + v][VD * (t / VE) + VE * c16 + (t % VE)] = o[t][v];
  __syncthreads();
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) {
    const int q = i / HD, dd = i - q * HD;
    float Mb = sm[0][q];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, sm[w][q]);
    if (DQ && owner) Mb = fmaxf(Mb, dq_s[q]);
    float v = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = (Mb == -INFINITY || sm[w][q] == -INFINITY) ? 0.f : exp2f(sm[w][q] - Mb);
      v = fmaf(f, so[w][q][dd], v);
      Ls = fmaf(f, sl[w][q], Ls);
    }
    if (DQ && owner) {  // the new row, weight 2^(score - reference)
      const float fn = exp2f(dq_s[q] - Mb);
      v = fmaf(fn, dq_kv[HD + dd], v);
      Ls += fn;
    }
    const int h = kvh * G + q;
    if (direct) {
      a.out[(size_t)h * HD + dd] = v / Ls;
    } else {
      part_o[((size_t)h * S + s) * HD + dd] = v;
      if (dd == 0) {
        part_ml[((size_t)h * S + s) * 2 + 0] = Mb;
        part_ml[((size_t)h * S + s) * 2 + 1] = Ls;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Verify-window attention in k_attn_mfma's form: 16-row tiles, each wave keeping
// its next kMfmaRing tiles' loads in flight, S^T on 16x16x32 and O += P V on
// 16x16x16, for the 16 query vectors of a query group (as k_attn_mid_mfma: vector
// j = qg * 16 + c16 over (m, g), m-major; query row m sees rows 0 .. ctx + m).
// fp32 K and V enter as bf16 (hi, lo) pairs (hi*hi + hi*lo + lo*hi summed, 2^-18
// relative); bf16 K and V are exact and only the queries and P are split.
template <int HD, typename KT>
__global__ __launch_bounds__(256, 2) void k_attn_vr(VerifyArgs a, int chunk, int S, int QG) {
  constexpr bool F32 = sizeof(KT) == 4;
  constexpr int NT = HD / 16;
  constexpr int KS = HD / 32;
  constexpr int VE0 = 16 / int(sizeof(KT));  // elements per 16-byte V load
  constexpr int VE = VE0 < NT ? VE0 : NT;
  constexpr int VD = 16 * VE;
  constexpr int NG = HD / VD;
  constexpr int KV = F32 ? 2 : 1;            // 16-byte K loads per k step
  constexpr int R = F32 ? 1 : kMfmaRing;     // fp32 tiles take twice the registers
  constexpr int STRIDE = 16 * kAttnWaves;
  static_assert(NT * 16 == HD && KS * 32 == HD && NG * VD == HD, "head_dim 64 or 128");
  __shared__ float so[kAttnWaves][16][HD + 4];
  __shared__ float sm[kAttnWaves][16], sl[kAttnWaves][16];

  const int nkv = a.n_head_kv, G = a.n_head / nkv;
  const int tiles = S * nkv;
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int tile = (slot / QG) * 8 + xcd, qg = slot % QG;
  if (tile >= tiles) return;
  const int s = tile % S, kvh = tile / S;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int T = a.ctx + a.M;
  const int r0 = s * chunk, r1 = min(T, r0 + chunk);
  const int rlast = r1 - 1;
  const KT* Kb = static_cast<const KT*>(a.k) + (size_t)kvh * a.cap * HD;
  const KT* Vb = static_cast<const KT*>(a.v) + (size_t)kvh * a.cap * HD;

  uint4 kr[R][KS][KV];
  uint4 vr[R][NG][4];
  auto load = [&](int i, int tb) {
    const KT* kp = Kb + (size_t)min(tb + c16, rlast) * HD + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int h = 0; h < KV; ++h) kr[i][ks][h] = *reinterpret_cast<const uint4*>(kp + 32 * ks + 4 * h);
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const KT* vp = Vb + (size_t)min(tb + 4 * g4 + v, rlast) * HD + VD * grp + VE * c16;
        if constexpr (VE * sizeof(KT) == 16) {
          vr[i][grp][v] = *reinterpret_cast<const uint4*>(vp);
        } else {  // 4 bf16 (head_dim 64)
          const uint2 w = *reinterpret_cast<const uint2*>(vp);
          vr[i][grp][v] = make_uint4(w.x, w.y, 0u, 0u);
        }
      }
  };
  const int tb0 = r0 + 16 * wv;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (tb0 + i * STRIDE < r1) load(i, tb0 + i * STRIDE);

  // this lane's query vector (S layout)
  const int jq = qg * 16 + c16, mq = jq / G;
  const bool qok = mq < a.M;
  const int lim = qok ? a.ctx + mq : -1;
  const int qrow = qok ? mq * a.n_head + kvh * G + (jq - mq * G) : 0;
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  bf16x8_t qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float* qp = a.q + (size_t)qrow * HD + 32 * ks + 8 * g4;
    const float4 u = *reinterpret_cast<const float4*>(qp), w = *reinterpret_cast<const float4*>(qp + 4);
    float x[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = qok ? x[e] * scale : 0.f;
    split8(x, qh[ks], ql[ks]);
  }
  f32x4_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  auto step = [&](int i, int tb) {
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (F32) {
        const uint4 u = kr[i][ks][0], w = kr[i][ks][1];
        const float x[8] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                            __uint_as_float(u.w), __uint_as_float(w.x), __uint_as_float(w.y),
                            __uint_as_float(w.z), __uint_as_float(w.w)};
        bf16x8_t kh, kl;
        split8(x, kh, kl);
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[ks], st, 0, 0, 0);
      } else {
        const bf16x8_t kh = __builtin_bit_cast(bf16x8_t, kr[i][ks][0]);
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], st, 0, 0, 0);
      }
    }
    uint4 vv[NG][4];
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
      for (int v = 0; v < 4; ++v) vv[grp][v] = vr[i][grp][v];
    if (tb + R * STRIDE < r1) load(i, tb + R * STRIDE);
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = tb + 4 * g4 + v;
      sc[v] = (row < r1 && row <= lim) ? st[v] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float fo = 1.f;
    if (mx > m + kRescale) {
      fo = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
      m = mx;
    }
    float pr[4], ps = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pr[v] = sc[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[v] - m);
      ps += pr[v];
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l = l * fo + ps;
    if (__any(fo != 1.f)) {
      float fv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) fv[v] = __shfl(fo, 4 * g4 + v, kWave);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[t][v] *= fv[v];
    }
    bf16x4s_t ph, pl;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const __bf16 h = (__bf16)pr[v];
      ph[v] = __builtin_bit_cast(short, h);
      pl[v] = __builtin_bit_cast(short, (__bf16)(pr[v] - (float)h));
    }
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
      for (int k = 0; k < VE; ++k) {
        const int t = VE * grp + k;
        if constexpr (F32) {
          bf16x4s_t vh, vl;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint4 w = vv[grp][v];
            const float x = __uint_as_float(k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w);
            const __bf16 h = (__bf16)x;
            vh[v] = __builtin_bit_cast(short, h);
            vl[v] = __builtin_bit_cast(short, (__bf16)(x - (float)h));
          }
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vh, o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vl, o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vh, o[t], 0, 0, 0);
        } else {
          bf16x4s_t vk;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint4 w = vv[grp][v];
            const uint32_t word = k < 2 ? w.x : k < 4 ? w.y : k < 6 ? w.z : w.w;
            vk[v] = (k & 1) ? short(word >> 16) : short(word & 0xffffu);
          }
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vk, o[t], 0, 0, 0);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vk, o[t], 0, 0, 0);
        }
      }
  };
  int tb = tb0;
  for (; tb + (R - 1) * STRIDE < r1; tb += R * STRIDE) {
#pragma unroll
    for (int i = 0; i < R; ++i) step(i, tb + i * STRIDE);
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (tb + i * STRIDE < r1) step(i, tb + i * STRIDE);

  if (g4 == 0) {
    sm[wv][c16] = m;
    sl[wv][c16] = l;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) so[wv][4 * g4 + v][VD * (t / VE) + VE * c16 + (t % VE)] = o[t][v];
  __syncthreads();
  const bool direct = S == 1;
  for (int i = threadIdx.x; i < 16 * HD; i += blockDim.x) {
    const int q = i / HD, dd = i - q * HD;
    const int j = qg * 16 + q, mm = j / G;
    if (mm >= a.M) continue;
    const int qr = mm * a.n_head + kvh * G + (j - mm * G);
    float Mb = sm[0][q];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, sm[w][q]);
    float v = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = (Mb == -INFINITY || sm[w][q] == -INFINITY) ? 0.f : exp2f(sm[w][q] - Mb);
      v = fmaf(f, so[w][q][dd], v);
      Ls = fmaf(f, sl[w][q], Ls);
    }
    if (direct) {
      a.out[(size_t)qr * HD + dd] = v / Ls;
    } else {
      a.part_o[((size_t)qr * S + s) * HD + dd] = v;
      if (dd == 0) {
        a.part_ml[((size_t)qr * S + s) * 2 + 0] = Mb;
        a.part_ml[((size_t)qr * S + s) * 2 + 1] = Ls;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_attn over quantized regions (q8_0 K, q5_1 V; layout in kernels.hpp).  A lane
// holds 8 consecutive K dims of a row, inside one block of 32, and the 8 V dims whose
// codes sit in the lane's 4 nibble bytes (and its high-bit byte): per row it loads 8
// K codes, its K block's scale, 4 bytes of V nibbles, the byte of V high bits and the
// (D, M) of the V blocks those dims fall in.  The K dot product is
// D_k * (sum_e code_e q_e - 128 sum_e q_e) (codes are stored + 128, sum_e q_e per lane
// precomputed); V values are D_v q + M_v.  The block whose split holds row T - 1
// first quantizes that row from kv_new into the cache (other blocks never read it).
// The MFMA kernel below (k_attn_qm) covers head_dim 64 and 128; this one the rest.
// Quantize the new row T - 1 of KV head kvh from kv_new into the cache (K dims then V
// dims, one per thread; the V codes are packed through LDS), visible to the whole
// block on return.  Every thread of the block calls it.
template <int HD>
__device__ __forceinline__ void quantize_new_row(const AttnArgs& a, int kvh) {
  __shared__ uint8_t vcode[HD];
  uint8_t* kreg = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
  uint8_t* vreg = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
  const int nkv = a.n_head_kv;
  const KvqAt at(nkv, a.cap, HD, kvh, a.T - 1);
  for (int i0 = 0; i0 < 2 * HD; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    const bool on = i < 2 * HD;  // whole groups of 32
    const bool is_k = i < HD;
    const int dim = is_k ? i : i - HD;
    const float x = on ? a.kv_new[(is_k ? 0 : nkv * HD) + kvh * HD + dim] : 0.f;
    const uint32_t q = kvq_quant(x, is_k, dim, kreg, vreg, at, on);
    if (on && !is_k) vcode[dim] = uint8_t(q);
  }
  __syncthreads();
  kvq_pack_v(vcode, HD, vreg, at, threadIdx.x, blockDim.x);
  __threadfence();
  __syncthreads();
}

template <int HD, int G>
__global__ __launch_bounds__(256) void k_attn_q(AttnArgs a, int chunk, int S) {
  constexpr int LPR = HD / kAttnLaneElems;  // lanes per row
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * kAttnWaves;
  constexpr int kDepth = 4;
  constexpr int NB = HD / 32;
  __shared__ float obuf[kAttnWaves][G][HD];
  __shared__ float s_M[kAttnWaves][G], s_L[kAttnWaves][G];

  const int s = blockIdx.x, kvh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int T = a.T, nkv = a.n_head_kv, cap = a.cap;
  const int r0 = s * chunk, r1 = min(T, r0 + chunk);
  if (r0 >= T) return;
  const uint8_t* kreg = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vreg = static_cast<const uint8_t*>(a.v_cache);
  if (a.kv_new && r1 == T) quantize_new_row<HD>(a, kvh);
  const bool direct = S == 1;
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  // per-lane bases: row r of this head at kc + r * HD etc.
  const size_t hr0 = (size_t)kvh * cap, all = (size_t)nkv * cap;
  const uint8_t* kc = kreg + hr0 * HD + sub * 8;
  const uint8_t* ks = kreg + all * HD + hr0 * (HD / 32) * 2 + (sub >> 2) * 2;
  const uint8_t* vn = vreg + hr0 * (HD / 2) + sub * 4;
  const uint8_t* vh = vreg + all * (HD / 2) + hr0 * (HD / 8) + sub;
  // the (D, M) of the V blocks of the lane's nibble bytes 4 sub + j: block (4 sub + j) % NB
  constexpr int NDM = NB < 4 ? NB : 4;
  const uint8_t* vd = vreg + all * (HD / 2 + HD / 8) + hr0 * NB * 4 + ((4 * sub) % NB) * 4;

  const int off = wv * RPW + slot;
  const int rlast = r1 - 1;
  uint2 kq[kDepth];
  uint32_t kd[kDepth], vq[kDepth], vb[kDepth], vm[kDepth][NDM];
  auto load_row = [&](int i, int row) {
    row = min(row, rlast);
    kq[i] = *reinterpret_cast<const uint2*>(kc + (size_t)row * HD);
    kd[i] = *reinterpret_cast<const uint16_t*>(ks + (size_t)row * (HD / 32) * 2);
    vq[i] = *reinterpret_cast<const uint32_t*>(vn + (size_t)row * (HD / 2));
    vb[i] = vh[(size_t)row * (HD / 8)];
    const uint8_t* dp = vd + (size_t)row * NB * 4;
    if constexpr (NDM == 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(dp);
      vm[i][0] = w.x; vm[i][1] = w.y; vm[i][2] = w.z; vm[i][3] = w.w;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(dp);
      vm[i][0] = w.x; vm[i][1] = w.y;
    }
  };
  int rb = r0;
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load_row(i, rb + off + i * RPB);
  float qv[G][kAttnLaneElems], qs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qs[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) {
      qv[g][e] = a.q[(size_t)(kvh * G + g) * HD + sub * 8 + e] * scale;
      qs[g] += qv[g][e];
    }
    qs[g] *= -128.f;
  }
  float m[G], mr[G], l[G], acc[G][kAttnLaneElems];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    mr[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] = 0.f;
  }
  auto step = [&](int i, int row) {
    // K codes (stored + 128) and V codes (low nibbles; the high bits moved to bit 4
    // of each byte: byte j of (b & mask) + (0x80 - 2^j) carries bit j into bit 7)
    uint32_t k0 = kq[i].x, k1 = kq[i].y;
    uint32_t nb = vq[i];
    const uint32_t hr = vb[i] * 0x01010101u;
    asm volatile("" : "+v"(k0), "+v"(k1), "+v"(nb));  // one v_cvt_f32_ubyteN per byte
    const uint32_t c_lo = (nb & 0x0F0F0F0Fu) | ((((hr & 0x08040201u) + 0x787C7E7Fu) & 0x80808080u) >> 3);
    const uint32_t c_hi = ((nb >> 4) & 0x0F0F0F0Fu) | ((((hr & 0x80402010u) + 0x00406070u) & 0x80808080u) >> 3);
    const float Dk = f16_bits_to_f32(uint16_t(kd[i]));
    const float kf[8] = {float(k0 & 0xFFu), float((k0 >> 8) & 0xFFu), float((k0 >> 16) & 0xFFu), float(k0 >> 24),
                         float(k1 & 0xFFu), float((k1 >> 8) & 0xFFu), float((k1 >> 16) & 0xFFu), float(k1 >> 24)};
    const float vc[8] = {float(c_lo & 0xFFu), float((c_lo >> 8) & 0xFFu), float((c_lo >> 16) & 0xFFu), float(c_lo >> 24),
                         float(c_hi & 0xFFu), float((c_hi >> 8) & 0xFFu), float((c_hi >> 16) & 0xFFu), float(c_hi >> 24)};
    // V values: byte j's two codes fall in block (4 sub + j) % NB
    float vf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = vm[i][j % NDM];
      const float Dv = f16_bits_to_f32(uint16_t(w & 0xFFFFu)), Mv = f16_bits_to_f32(uint16_t(w >> 16));
      vf[j] = fmaf(Dv, vc[j], Mv);
      vf[j + 4] = fmaf(Dv, vc[j + 4], Mv);
    }
    load_row(i, row + kDepth * RPB);
    float d[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float t = qs[g];
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) t = fmaf(kf[e], qv[g][e], t);
      d[g] = t * Dk;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) d[g] = group_sum<LPR>(d[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = d[g];
      if (sc > mr[g]) {
        const float fo = __builtin_amdgcn_exp2f(m[g] - sc);
        l[g] *= fo;
#pragma unroll
        for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] *= fo;
        m[g] = sc;
        mr[g] = sc + kRescale;
      }
      const float p = __builtin_amdgcn_exp2f(sc - m[g]);
      l[g] += p;
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  };
  for (; rb + kDepth * RPB <= r1; rb += kDepth * RPB) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) step(i, rb + off + i * RPB);
  }
  if (rb < r1) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      const int rr = rb + off + i * RPB;
      if (rr >= r1) break;
      step(i, rr);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mw = wave_max(m[g]);
    if (lane == 0) s_M[wv][g] = mw;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float Mb = s_M[0][g];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, s_M[w][g]);
    const float f = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - Mb);
    l[g] *= f;
#pragma unroll
    for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] *= f;
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] += __shfl_xor(l[g], o, kWave);
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) acc[g][e] += __shfl_xor(acc[g][e], o, kWave);
    }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < kAttnLaneElems; ++e) obuf[wv][g][vq_dim(4 * sub + (e & 3), e >> 2, HD)] = acc[g][e];
      if (sub == 0) s_L[wv][g] = l[g];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) {
    const int g = i / HD, dd = i - g * HD;
    float v = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      v += obuf[w][g][dd];
      L += s_L[w][g];
    }
    const int h = kvh * G + g;
    if (direct) a.out[(size_t)h * HD + dd] = v / L;
    else a.part_o[((size_t)h * S + s) * HD + dd] = v;
  }
  if (direct) return;
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float Mb = s_M[0][g], L = 0.f;
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, s_M[w][g]);
    for (int w = 0; w < kAttnWaves; ++w) L += s_L[w][g];
    const int h = kvh * G + g;
    a.part_ml[((size_t)h * S + s) * 2 + 0] = Mb;
    a.part_ml[((size_t)h * S + s) * 2 + 1] = L;
  }
}

// ---------------------------------------------------------------------------
// q8q5 decode attention on MFMA (head_dim 64 or 128, at most 16 query heads per KV
// head) over 16-row tiles.  Scores: per 32-dim block ks, S^T_ks = K_ks . Q^T on
// v_mfma_f32_16x16x32_f16 with the codes as fp16 1024 + u (u = the stored code + 128;
// one byte permute per two codes) against the queries as fp16 (hi, lo) pairs scaled
// by 2^e per query; the product's accumulator starts at -1152 sum_ks q, the block
// scales it by D_k, the sum over the blocks is scaled back by 2^-e.  Values: O^T =
// V^T P^T on v_mfma_f32_16x16x16bf16_1k, output tile t = (block b, half h) holding
// dims 32 b + 16 h + (0..15): A = the tile's codes over the 16 rows as bf16 128 + c, B
// = P^T with each row's weight times that row's D_v of block b, as bf16 (hi, lo); the
// block's M_v and the 128 offset give a per-(query, block) term sum_r p_r (M_v - 128
// D_v) added at the end.  The lane holding query c16's scores of rows 4 g4 + v is
// P^T's operand lane, and O^T's D layout keeps query c16 in the lane's column, so the
// online softmax rescales O in place.
//
// Each wave streams its own tiles through a ring of kQmRing LDS slots: a tile's five
// arrays (K codes, V nibbles, K scales, V high bits, V (D, M)) are contiguous runs of
// the head's region, read with global_load_lds (a lane's 16 bytes land at its lane
// slot of a 1 KB wave write), so kQmRing - 1 tiles are in flight without holding
// registers.  Lanes choose their source chunks so that the reads are spread over the
// LDS banks: chunk p of K row r holds the row's chunk p ^ (r % (hd / 16)); V nibble
// rows sit in the order 4 (r % 4) + r / 4.  Tiles past the chunk's last row read rows
// of the region beyond T (the region holds a multiple of 16 rows, zeroed at
// allocation, so they are finite) and are masked out of the softmax.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// ring depth: three slots (three blocks a CU by LDS; 32767 rows, 40/8 heads: 22.5 us
// against 23.7 with four slots and two blocks a CU); EAGLE3_QM_RING=4 for comparison
constexpr int kQmRing = 3;
// EAGLE3_QM_ODD=0 keeps the q8q5 kernel's split length as picked (for comparison)
static bool T_odd_steps() {
  static const bool v = [] {
    const char* e = std::getenv("EAGLE3_QM_ODD");
    return !(e && e[0] == '0');
  }();
  return v;
}
static int qm_ring() {
  static const int r = [] {
    const char* e = std::getenv("EAGLE3_QM_RING");
    return (e && e[0] == '4') ? 4 : kQmRing;
  }();
  return r;
}

// One lane's reads of a ring slot (LDS byte addresses), issued together and waited
// for in the same statement: the compiler does not see them as LDS reads that the
// ring's in-flight global_load_lds writes might alias (it would wait for every
// outstanding write before each); the ring's own vmcnt wait orders them, and the
// memory clobber keeps the slot's refill (issued after them) from moving above them.
// kc[ks]: the lane's 8 K code bytes of block ks (ak[ks]); ksc: the K scales of rows
// 4 g4 .. + 3 (as); vn[v], vh[v], dm[v]: the V nibbles, high-bit byte and (D, M) of
// row 4 g4 + v (an, ah, ad: row 4 g4's, in the slot's row orders).
__device__ __forceinline__ void qm_read(u32x2_t (&kc)[4], u32x4_t (&ksc)[2], uint32_t (&vn)[4], uint32_t (&vh)[4],
                                        u32x4_t (&dm)[4], const uint32_t (&ak)[4], uint32_t as, uint32_t an,
                                        uint32_t ah, uint32_t ad) {  // head_dim 128
  asm volatile(
      "ds_read_b64 %0, %18\n"
      "ds_read_b64 %1, %19\n"
      "ds_read_b64 %2, %20\n"
      "ds_read_b64 %3, %21\n"
      "ds_read_b128 %4, %22\n"
      "ds_read_b128 %5, %22 offset:16\n"
      "ds_read_b32 %6, %23\n"
      "ds_read_b32 %7, %23 offset:256\n"
      "ds_read_b32 %8, %23 offset:512\n"
      "ds_read_b32 %9, %23 offset:768\n"
      "ds_read_u8 %10, %24\n"
      "ds_read_u8 %11, %24 offset:16\n"
      "ds_read_u8 %12, %24 offset:32\n"
      "ds_read_u8 %13, %24 offset:48\n"
      "ds_read_b128 %14, %25\n"
      "ds_read_b128 %15, %25 offset:16\n"
      "ds_read_b128 %16, %25 offset:32\n"
      "ds_read_b128 %17, %25 offset:48\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kc[0]), "=&v"(kc[1]), "=&v"(kc[2]), "=&v"(kc[3]), "=&v"(ksc[0]), "=&v"(ksc[1]), "=&v"(vn[0]),
        "=&v"(vn[1]), "=&v"(vn[2]), "=&v"(vn[3]), "=&v"(vh[0]), "=&v"(vh[1]), "=&v"(vh[2]), "=&v"(vh[3]),
        "=&v"(dm[0]), "=&v"(dm[1]), "=&v"(dm[2]), "=&v"(dm[3])
      : "v"(ak[0]), "v"(ak[1]), "v"(ak[2]), "v"(ak[3]), "v"(as), "v"(an), "v"(ah), "v"(ad)
      : "memory");
}
__device__ __forceinline__ void qm_read(u32x2_t (&kc)[2], u32x4_t& ksc, uint32_t (&vn)[4], uint32_t (&vh)[4],
                                        u32x2_t (&dm)[4], const uint32_t (&ak)[2], uint32_t as, uint32_t an,
                                        uint32_t ah, uint32_t ad) {  // head_dim 64
  asm volatile(
      "ds_read_b64 %0, %15\n"
      "ds_read_b64 %1, %16\n"
      "ds_read_b128 %2, %17\n"
      "ds_read_u16 %3, %18\n"
      "ds_read_u16 %4, %18 offset:128\n"
      "ds_read_u16 %5, %18 offset:256\n"
      "ds_read_u16 %6, %18 offset:384\n"
      "ds_read_u8 %7, %19\n"
      "ds_read_u8 %8, %19 offset:8\n"
      "ds_read_u8 %9, %19 offset:16\n"
      "ds_read_u8 %10, %19 offset:24\n"
      "ds_read_b64 %11, %20\n"
      "ds_read_b64 %12, %20 offset:8\n"
      "ds_read_b64 %13, %20 offset:16\n"
      "ds_read_b64 %14, %20 offset:24\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kc[0]), "=&v"(kc[1]), "=&v"(ksc), "=&v"(vn[0]), "=&v"(vn[1]), "=&v"(vn[2]), "=&v"(vn[3]),
        "=&v"(vh[0]), "=&v"(vh[1]), "=&v"(vh[2]), "=&v"(vh[3]), "=&v"(dm[0]), "=&v"(dm[1]), "=&v"(dm[2]),
        "=&v"(dm[3])
      : "v"(ak[0]), "v"(ak[1]), "v"(as), "v"(an), "v"(ah), "v"(ad)
      : "memory");
}

template <int HD>
struct QmTile {
  static constexpr int NB = HD / 32;       // 32-dim blocks
  static constexpr int CPR = HD / 16;      // 16-byte chunks of a K row
  static constexpr int CPV = HD / 32;      // 16-byte chunks of a V nibble row
  // the arrays' first 16-byte chunk in a slot
  static constexpr int K = 0, VN = HD, KS = VN + HD / 2, VH = KS + 2 * NB, VD = VH + HD / 8, END = VD + 4 * NB;
  static constexpr int NI = (END + 63) / 64;  // 1 KB wave writes per tile
  static constexpr int BYTES = NI * 1024;
};

template <int HD, int D>
__global__ __launch_bounds__(256, D == 3 ? 3 : 2) void k_attn_qm(AttnArgs a, int chunk, int S) {
  using TL = QmTile<HD>;
  constexpr int NB = TL::NB;
  constexpr int NT = HD / 16;  // output tiles of O^T, t = 2 b + h
  constexpr int NI = TL::NI;
  constexpr int STRIDE = 16 * kAttnWaves;
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
  static_assert(kAttnWaves * 16 * (HD + 4) * 4 <= kAttnWaves * D * TL::BYTES, "the merge fits in the ring");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kAttnWaves * D * TL::BYTES];
  __shared__ float sm[kAttnWaves][16], sl[kAttnWaves][16];

  const int s = blockIdx.x, kvh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int G = a.n_head / a.n_head_kv;
  const int T = a.T, nkv = a.n_head_kv, cap = a.cap;
  const int r0 = s * chunk, r1 = min(T, r0 + chunk);
  if (r0 >= T) return;
  if (a.kv_new && r1 == T) quantize_new_row<HD>(a, kvh);
  const bool direct = S == 1;
  const uint8_t* kreg = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vreg = static_cast<const uint8_t*>(a.v_cache);
  const size_t hr0 = (size_t)kvh * cap, all = (size_t)nkv * cap;

  // this lane's source for each of the tile's NI wave writes: the chunk's address at
  // tile row 0 and the bytes per row of its array
  const uint8_t* src[NI];
  uint32_t rowb[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int c = 64 * k + lane;
    if (c < TL::VN) {  // K codes: row r, slot p <- chunk p ^ (r % CPR)
      const int r = c / TL::CPR, p = c % TL::CPR;
      src[k] = kreg + hr0 * HD + r * HD + 16 * (p ^ (r % TL::CPR));
      rowb[k] = HD;
    } else if (c < TL::KS) {  // V nibbles: slot row q holds row 4 (q % 4) + q / 4
      const int w = c - TL::VN, q = w / TL::CPV, p = w % TL::CPV;
      const int r = 4 * (q % 4) + q / 4;
      src[k] = vreg + hr0 * (HD / 2) + r * (HD / 2) + 16 * p;
      rowb[k] = HD / 2;
    } else if (c < TL::VH) {  // K scales
      src[k] = kreg + all * HD + hr0 * NB * 2 + 16 * (c - TL::KS);
      rowb[k] = NB * 2;
    } else if (c < TL::VD) {  // V high bits
      src[k] = vreg + all * (HD / 2) + hr0 * (HD / 8) + 16 * (c - TL::VH);
      rowb[k] = HD / 8;
    } else if (c < TL::END) {  // V (D, M)
      src[k] = vreg + all * (HD / 2 + HD / 8) + hr0 * NB * 4 + 16 * (c - TL::VD);
      rowb[k] = NB * 4;
    } else {  // past the tile's bytes: a K chunk into the slot's unused tail
      src[k] = kreg + hr0 * HD;
      rowb[k] = HD;
    }
  }
  uint8_t* wring = ring + wv * D * TL::BYTES;
  // tile k of this wave starts at row tb0 + k STRIDE and goes to slot k % D.  Every
  // step issues one tile D ahead, past the wave's last tile that tile again (a wave
  // without tiles takes the block's first), so exactly D - 1 tiles' writes are in
  // flight behind the one a step reads, and every lane takes part in every write.
  const int tb0 = r0 + 16 * wv;
  const int ntile = tb0 < r1 ? (r1 - tb0 + STRIDE - 1) / STRIDE : 0;
  // byte offsets of the chunks from kreg (a sequence's K and V regions span well under
  // 4 GiB), at the wave's first tile
  // (off: the next tile to issue; it advances by one wave step per tile up to the
  // wave's last tile; islot: that tile's slot)
  uint32_t off[NI], step[NI];
  const int tfirst = ntile > 0 ? tb0 : r0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    off[i] = uint32_t(src[i] - kreg) + uint32_t(tfirst) * rowb[i];
    step[i] = uint32_t(STRIDE) * rowb[i];
  }
  int islot = 0;
  auto issue = [&](int k) {
    uint8_t* dst = wring + islot * TL::BYTES;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(kreg + off[i]),
                                       (void __attribute__((address_space(3)))*)(dst + 1024 * i), 16, 0, 0);
    if (k < ntile - 1)
#pragma unroll
      for (int i = 0; i < NI; ++i) off[i] += step[i];
    islot = islot + 1 == D ? 0 : islot + 1;
  };

  // query c16's dims 32 ks + 8 g4 .. + 7 with the base-2 score scale, times 2^e
  // putting the query's largest value in [2^14, 2^15), as fp16 (hi, lo); columns
  // past G are zero.  qs[ks]: -1152 times the block's sum of (hi + lo) over its 32 dims.
  const float scale = 1.4426950408889634f / sqrtf(float(HD));
  const bool qok = c16 < G;
  float4 qv[NB][2];  // loaded before the ring's first tiles are issued
#pragma unroll
  for (int ks = 0; ks < NB; ++ks) {
    const float* qp = a.q + (size_t)(kvh * G + (qok ? c16 : 0)) * HD + 32 * ks + 8 * g4;
    qv[ks][0] = *reinterpret_cast<const float4*>(qp);
    qv[ks][1] = *reinterpret_cast<const float4*>(qp + 4);
  }
#pragma unroll
  for (int k = 0; k < D; ++k) issue(k);
  float x[NB][8];
  float amax = 0.f;
#pragma unroll
  for (int ks = 0; ks < NB; ++ks) {
    const float4 u = qv[ks][0], w = qv[ks][1];
    const float y[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[ks][e] = qok ? y[e] * scale : 0.f;
      amax = fmaxf(amax, fabsf(x[ks][e]));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  int ex = 0;
  if (amax > 0.f) (void)frexpf(amax, &ex);
  ex = max(ex, -100);  // 2^(15 - ex) stays finite
  const float up = ldexpf(1.f, 15 - ex), down = ldexpf(1.f, ex - 15);
  f16x8_t qh[NB], ql[NB];
  float qs[NB];
#pragma unroll
  for (int ks = 0; ks < NB; ++ks) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float yv = x[ks][e] * up;
      const _Float16 h = (_Float16)yv;
      const _Float16 lo = (_Float16)(yv - (float)h);
      qh[ks][e] = h;
      ql[ks][e] = lo;
      t += (float)h + (float)lo;
    }
    t += __shfl_xor(t, 16, kWave);
    t += __shfl_xor(t, 32, kWave);
    qs[ks] = -1152.f * t;
  }
  f32x4_t o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float cb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) cb[b] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int hsh = (c16 * NB) & 3;  // the lane's first bit in its high-bit byte
  // the lane's LDS byte offsets in a slot (qm_read)
  const uint32_t lds_w = uint32_t((uintptr_t)((__attribute__((address_space(3))) uint8_t*)wring));
  uint32_t ak[NB];
#pragma unroll
  for (int ks = 0; ks < NB; ++ks)
    ak[ks] = c16 * HD + 16 * ((2 * ks + (g4 >> 1)) ^ (c16 % TL::CPR)) + 8 * (g4 & 1);
  const uint32_t o_s = 16 * TL::KS + 4 * g4 * (NB * 2), o_n = 16 * TL::VN + g4 * (HD / 2) + c16 * NB,
                 o_h = 16 * TL::VH + 4 * g4 * (HD / 8) + ((c16 * NB) >> 2), o_d = 16 * TL::VD + 4 * g4 * (NB * 4);

  int rslot = 0;
  for (int k = 0; k < ntile; ++k) {
    // tile k has landed once at most the D - 1 later tiles' writes are outstanding
    wait_vmcnt<(D - 1) * NI>();
    const int tb = tb0 + k * STRIDE;
    const uint32_t sb = lds_w + uint32_t(rslot * TL::BYTES);
    rslot = rslot + 1 == D ? 0 : rslot + 1;
    u32x2_t kc[NB];
    uint32_t kd[4][(NB + 1) / 2], vn[4], vh[4], dm[4][NB];
    uint32_t aks[NB];
#pragma unroll
    for (int ks = 0; ks < NB; ++ks) aks[ks] = sb + ak[ks];
    if constexpr (NB == 4) {
      u32x4_t ksc[2], dmv[4];
      qm_read(kc, ksc, vn, vh, dmv, aks, sb + o_s, sb + o_n, sb + o_h, sb + o_d);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        kd[v][0] = (v & 1) ? ksc[v >> 1].z : ksc[v >> 1].x;
        kd[v][1] = (v & 1) ? ksc[v >> 1].w : ksc[v >> 1].y;
#pragma unroll
        for (int b = 0; b < NB; ++b) dm[v][b] = dmv[v][b];
      }
    } else {
      u32x4_t ksc;
      u32x2_t dmv[4];
      qm_read(kc, ksc, vn, vh, dmv, aks, sb + o_s, sb + o_n, sb + o_h, sb + o_d);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        kd[v][0] = ksc[v];
#pragma unroll
        for (int b = 0; b < NB; ++b) dm[v][b] = dmv[v][b];
      }
    }
    // scores of rows tb + 4 g4 + v for query c16 (times 2^e)
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NB; ++ks) {
      const u32x2_t kq = kc[ks];
      const uint32_t e4 = 0x64646464u;  // fp16 1024 + u: high byte 0x64 over the code
      uint4 av;
      av.x = __builtin_amdgcn_perm(e4, kq.x, 0x04010400u);
      av.y = __builtin_amdgcn_perm(e4, kq.x, 0x04030402u);
      av.z = __builtin_amdgcn_perm(e4, kq.y, 0x04010400u);
      av.w = __builtin_amdgcn_perm(e4, kq.y, 0x04030402u);
      const f16x8_t ka = __builtin_bit_cast(f16x8_t, av);
      f32x4_t st = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qh[ks], f32x4_t{qs[ks], qs[ks], qs[ks], qs[ks]}, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, ql[ks], st, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t w = kd[v][ks >> 1];
        const float Dk = f16_bits_to_f32(uint16_t((ks & 1) ? (w >> 16) : (w & 0xFFFFu)));
        acc[v] = fmaf(Dk, st[v], acc[v]);
      }
    }
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = (tb + 4 * g4 + v < r1) ? acc[v] * down : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float fo = 1.f;
    if (mx > m + kRescale) {
      fo = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
      m = mx;
    }
    float pr[4], ps = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pr[v] = sc[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[v] - m);
      ps += pr[v];
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l = l * fo + ps;
    if (__any(fo != 1.f)) {  // O^T's D layout: the lane's column is query c16
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[t][v] *= fo;
#pragma unroll
      for (int b = 0; b < NB; ++b) cb[b] *= fo;
    }
    // V codes: byte b of clo / chi = the code of dim 32 b + c16 / 32 b + 16 + c16
    uint32_t clo[4], chi[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t nb = vn[v];
      const uint32_t hr = ((vh[v] >> hsh) & 0xFFu) * 0x01010101u;
      clo[v] = (nb & 0x0F0F0F0Fu) | ((((hr & 0x08040201u) + 0x787C7E7Fu) & 0x80808080u) >> 3);
      chi[v] = ((nb >> 4) & 0x0F0F0F0Fu) | ((((hr & 0x80402010u) + 0x00406070u) & 0x80808080u) >> 3);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // P^T for block b: each row's weight times its D_v, as bf16 (hi, lo), converted
      // two values an instruction
      f32x4_t pv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float Dv = f16_bits_to_f32(uint16_t(dm[v][b] & 0xFFFFu));
        const float Mv = f16_bits_to_f32(uint16_t(dm[v][b] >> 16));
        pv[v] = pr[v] * Dv;
        cb[b] = fmaf(pr[v], fmaf(-128.f, Dv, Mv), cb[b]);
      }
      const f32x2_t p01 = {pv[0], pv[1]}, p23 = {pv[2], pv[3]};
      const bf16x2_t h01 = __builtin_convertvector(p01, bf16x2_t), h23 = __builtin_convertvector(p23, bf16x2_t);
      const bf16x2_t l01 = __builtin_convertvector(p01 - __builtin_convertvector(h01, f32x2_t), bf16x2_t);
      const bf16x2_t l23 = __builtin_convertvector(p23 - __builtin_convertvector(h23, f32x2_t), bf16x2_t);
      const bf16x4s_t ph = __builtin_bit_cast(bf16x4s_t, u32x2_t{__builtin_bit_cast(uint32_t, h01),
                                                                  __builtin_bit_cast(uint32_t, h23)});
      const bf16x4s_t pl = __builtin_bit_cast(bf16x4s_t, u32x2_t{__builtin_bit_cast(uint32_t, l01),
                                                                  __builtin_bit_cast(uint32_t, l23)});
      const uint32_t sel = uint32_t(b) | (0x0Cu << 8) | (uint32_t(4 + b) << 16) | (0x0Cu << 24);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t* X = hh ? chi : clo;
        uint2 w;
        w.x = __builtin_amdgcn_perm(X[1], X[0], sel) | 0x43004300u;  // rows 0, 1 as bf16 128 + c
        w.y = __builtin_amdgcn_perm(X[3], X[2], sel) | 0x43004300u;  // rows 2, 3
        const bf16x4s_t av = __builtin_bit_cast(bf16x4s_t, w);
        const int t = 2 * b + hh;
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, ph, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pl, o[t], 0, 0, 0);
      }
    }
    // the slot is free once every lane's reads of it are done
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    issue(k + D);
  }
  wait_vmcnt<0>();  // the ring's last writes have landed before it turns into the merge buffer

  // the per-(query, block) terms over the lane group's rows, then the waves merge
  // (the merge buffer takes the ring's place once every wave is done with it)
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    cb[b] += __shfl_xor(cb[b], 16, kWave);
    cb[b] += __shfl_xor(cb[b], 32, kWave);
  }
  if (g4 == 0) {
    sm[wv][c16] = m;
    sl[wv][c16] = l;
  }
  __syncthreads();
  float(*so)[16][HD + 4] = reinterpret_cast<float(*)[16][HD + 4]>(ring);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) so[wv][c16][16 * t + 4 * g4 + v] = o[t][v] + cb[t >> 1];
  __syncthreads();
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) {
    const int q = i / HD, dd = i - q * HD;
    float Mb = sm[0][q];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) Mb = fmaxf(Mb, sm[w][q]);
    float v = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = (Mb == -INFINITY || sm[w][q] == -INFINITY) ? 0.f : exp2f(sm[w][q] - Mb);
      v = fmaf(f, so[w][q][dd], v);
      Ls = fmaf(f, sl[w][q], Ls);
    }
    const int h = kvh * G + q;
    if (direct) {
      a.out[(size_t)h * HD + dd] = v / Ls;
    } else {
      a.part_o[((size_t)h * S + s) * HD + dd] = v;
      if (dd == 0) {
        a.part_ml[((size_t)h * S + s) * 2 + 0] = Mb;
        a.part_ml[((size_t)h * S + s) * 2 + 1] = Ls;
      }
    }
  }
}

// One block of hd threads per query head: o = sum_s w_s o_s with
// w_s = 2^(m_s - M) / sum_z l_z 2^(m_z - M) (m in base 2, M the largest m_s).
// Splits are taken kCombineRegs at a time: this thread's column of the group's
// partial outputs and (wave 0, lane z) split z's (m, l) are loaded together, so
// up to kCombineRegs splits cost one memory round trip; the maximum and the
// weighted sum of l are wave reductions, the weights shared through LDS.
constexpr int kCombineRegs = 64;

__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int S,
                                                      int hd, float* __restrict__ out) {
  __shared__ float sw[kCombineRegs];
  __shared__ float sL[1];
  const int h = blockIdx.x, d = threadIdx.x;
  const int lane = d & 63, wv = d >> 6;
  const float* ml = part_ml + (size_t)h * S * 2;
  const float* po = part_o + (size_t)h * S * hd + d;
  float acc = 0.f, Lsum = 0.f, M = -INFINITY;
  for (int z0 = 0; z0 < S; z0 += kCombineRegs) {
    const int cnt = min(kCombineRegs, S - z0);
    float o[kCombineRegs];
#pragma unroll
    for (int i = 0; i < kCombineRegs; ++i) o[i] = i < cnt ? po[(size_t)(z0 + i) * hd] : 0.f;
    float mz = -INFINITY, lz = 0.f;
    if (wv == 0 && lane < cnt) {
      mz = ml[2 * (z0 + lane)];
      lz = ml[2 * (z0 + lane) + 1];
    }
    if (wv == 0) {
      if (z0 == 0) {  // the maximum over all splits
        float mm = mz;
        for (int z = kCombineRegs + lane; z < S; z += 64) mm = fmaxf(mm, ml[2 * z]);
        M = wave_max(mm);
      }
      if (lane < cnt) {
        const float e = exp2f(mz - M);
        sw[lane] = e;
        Lsum = fmaf(e, lz, Lsum);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCombineRegs; ++i)
      if (i < cnt) acc = fmaf(sw[i], o[i], acc);
    __syncthreads();
  }
  if (wv == 0) {
    Lsum = wave_sum(Lsum);
    if (lane == 0) sL[0] = Lsum;
  }
  __syncthreads();
  if (d < hd) out[(size_t)h * hd + d] = acc / sL[0];
}

// Batched combine: grid (n_head, rows); row r has ceil(T_r / chunk) splits of the
// Smax-strided partials.  Output as bf16 (hi, lo) pairs [row][ld].
__global__ __launch_bounds__(128) void k_attn_combine_b(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml, int Smax,
                                                        int hd, int n_head, int chunk, int step,
                                                        const BatchRows br,
                                                        uint16_t* __restrict__ out_hi,
                                                        uint16_t* __restrict__ out_lo, int ld) {
  extern __shared__ float w[];  // [Smax]
  __shared__ float red[32];
  const int h = blockIdx.x, r = blockIdx.y;
  const int T = br.row0[r] + step + 1;
  const int S = (T + chunk - 1) / chunk;
  const float* ml = part_ml + ((size_t)r * n_head + h) * Smax * 2;
  float M = -INFINITY;
  for (int z = threadIdx.x; z < S; z += blockDim.x) M = fmaxf(M, ml[2 * z]);
  M = wave_max(M);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) red[wv] = M;
  __syncthreads();
  M = red[0];
  for (int k = 1; k < nw; ++k) M = fmaxf(M, red[k]);
  float L = 0.f, dummy = 0.f;
  for (int z = threadIdx.x; z < S; z += blockDim.x) {
    const float e = exp2f(ml[2 * z] - M);
    w[z] = e;
    L = fmaf(e, ml[2 * z + 1], L);
  }
  __syncthreads();
  block_sum2(L, dummy, red);
  const float invL = 1.0f / L;
  const float* po = part_o + ((size_t)r * n_head + h) * Smax * hd;
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float acc0 = 0.f, acc1 = 0.f;
    int z = 0;
    for (; z + 1 < S; z += 2) {
      acc0 = fmaf(w[z], po[(size_t)z * hd + d], acc0);
      acc1 = fmaf(w[z + 1], po[(size_t)(z + 1) * hd + d], acc1);
    }
    if (z < S) acc0 = fmaf(w[z], po[(size_t)z * hd + d], acc0);
    const float o = (acc0 + acc1) * invL;
    const uint16_t hi = f32_to_bf16(o);
    const size_t at = (size_t)r * ld + (size_t)h * hd + d;
    out_hi[at] = hi;
    out_lo[at] = f32_to_bf16(o - bf16_to_f32(hi));
  }
}

static inline int rows_per_block(int hd, int kv_f32) {
  (void)kv_f32;
  return kAttnWaves * (64 / (hd / kAttnLaneElems));
}

// (kv head, split) blocks aimed at by the single-row attention; EAGLE3_ATTN_BLOCKS
// overrides it (8..512) for tuning
static int attn_single_blocks() {
  static const int t = [] {
    const char* e = std::getenv("EAGLE3_ATTN_BLOCKS");
    const int v = e ? std::atoi(e) : 0;
    return (v >= 8 && v <= 512) ? v : kAttnSingleBlocks;
  }();
  return t;
}

// A power-of-two split length of the VALU decode kernel grows by one row block: then
// not every block's reads start at the same power-of-two offsets (32767 fp32 rows,
// 40/8 heads: 47.5 against 49.1 us with 512-row splits; the bf16 MFMA kernel showed no
// difference).  EAGLE3_ATTN_ODD=0 keeps the power of two.
static bool attn_odd() {
  static const bool v = [] {
    const char* e = std::getenv("EAGLE3_ATTN_ODD");
    return !(e && e[0] == '0');
  }();
  return v;
}

static void pick_split(int T, int n_head_kv, int hd, int kv_f32, int* chunk, int* S, int blocks = 0,
                       int rpb = 0) {
  if (rpb <= 0) rpb = rows_per_block(hd, kv_f32);
  if (blocks <= 0) blocks = attn_single_blocks();
  const int target = n_head_kv >= blocks ? 1 : blocks / n_head_kv;
  int c = (T + target - 1) / target;
  c = ((c + rpb - 1) / rpb) * rpb;
  if (c < rpb) c = rpb;
  if (c > kAttnMaxChunk) c = kAttnMaxChunk;
  if (attn_odd() && (c & (c - 1)) == 0 && c >= 256 && c < T) c += rpb;
  *chunk = c;
  *S = (T + c - 1) / c;
}

// Splits of the MFMA decode kernel: about kAttnSingleBlocks (KV head, split) blocks,
// chunks of whole 16-row tiles per wave (64 rows), at most kAttnMfmaMaxChunk rows;
// longer chunks than the VALU kernel's, since a block's fixed work (queries, merge)
// is larger (at 32K rows over 8 KV heads: 1024-row chunks 23.7 us, 512 27.8, 256 35.2)

static void pick_split_mfma(int T, int n_head_kv, int* chunk, int* S, int blocks = 0) {
  if (blocks <= 0) blocks = attn_single_blocks();
  const int target = n_head_kv >= blocks ? 1 : blocks / n_head_kv;
  constexpr int rpb = 16 * kAttnWaves;
  int c = (T + target - 1) / target;
  c = ((c + rpb - 1) / rpb) * rpb;
  if (c < rpb) c = rpb;
  if (c > kAttnMfmaMaxChunk) c = kAttnMfmaMaxChunk;
  *chunk = c;
  *S = (T + c - 1) / c;
}

int attn_max_splits(int cap, int head_dim, int n_head_kv) {
  // S = ceil(T / chunk) never exceeds the target split count while chunks are
  // uncapped, nor ceil(T / kAttnMaxChunk) once they are capped
  (void)head_dim;
  const int target = n_head_kv >= 512 ? 1 : 512 / n_head_kv;
  const int capped = (cap + kAttnMaxChunk - 1) / kAttnMaxChunk;
  return (target > capped ? target : capped) + 1;
}

// EAGLE3_ATTN_VALU=1 keeps bf16 decode attention on the VALU kernel (for comparison)
static bool attn_valu() {
  static const bool v = [] {
    const char* e = std::getenv("EAGLE3_ATTN_VALU");
    return e && e[0] == '1';
  }();
  return v;
}

// bf16 K/V at head_dim <= 128 with at most 16 query heads per KV head run k_attn_mfma
static bool attn_on_mfma(int hd, int kv_f32, int G) { return !kv_f32 && hd <= 128 && G <= 16 && !attn_valu(); }

template <int HD, typename KT>
static hipError_t launch_hd(const AttnArgs& a, int G, int chunk, int S, hipStream_t s,
                            int rows = 1) {
  dim3 grid(S, a.n_head_kv, rows), block(64 * kAttnWaves);
  if constexpr (sizeof(KT) == 2 && HD <= 128) {
    if (attn_on_mfma(HD, 0, G)) {
      if (a.dq) hipLaunchKernelGGL((k_attn_mfma<HD, true>), grid, block, 0, s, a, chunk, S);
      else hipLaunchKernelGGL((k_attn_mfma<HD, false>), grid, block, 0, s, a, chunk, S);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || S == 1 || a.batched) return e;
      hipLaunchKernelGGL(k_attn_combine, dim3(a.n_head), dim3(HD), 0, s, a.part_o, a.part_ml, S, HD,
                         a.out);
      return hipGetLastError();
    }
  }
#define E3_ATTN_CASE(GG)                                                                  \
  case GG:                                                                              \
    if (a.dq) hipLaunchKernelGGL((k_attn<HD, GG, KT, true>), grid, block, 0, s, a, chunk, S); \
    else hipLaunchKernelGGL((k_attn<HD, GG, KT, false>), grid, block, 0, s, a, chunk, S);      \
    break;
  switch (G) {
    E3_ATTN_CASE(1)
    E3_ATTN_CASE(2)
    E3_ATTN_CASE(3)
    E3_ATTN_CASE(4)
    E3_ATTN_CASE(5)
    E3_ATTN_CASE(6)
    E3_ATTN_CASE(7)
    E3_ATTN_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef E3_ATTN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1 || a.batched) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(a.n_head), dim3(HD), 0, s, a.part_o, a.part_ml, S, HD,
                     a.out);
  return hipGetLastError();
}

template <typename KT>
static hipError_t launch_kt(const AttnArgs& a, int G, int chunk, int S, hipStream_t s,
                            int rows = 1) {
  switch (a.head_dim) {
    case 64: return launch_hd<64, KT>(a, G, chunk, S, s, rows);
    case 128: return launch_hd<128, KT>(a, G, chunk, S, s, rows);
    case 256: return launch_hd<256, KT>(a, G, chunk, S, s, rows);
    default: return hipErrorInvalidValue;
  }
}

// Batched rows share one chunk size: about attn_batch_target() (row, head, split)
// blocks in total, between kAttnBatchMinChunk and kAttnMaxChunk rows per split.
constexpr int kAttnBatchMinChunk = 128;

// (row, head, split) blocks aimed at per batched launch; EAGLE3_ATTN_BATCH_BLOCKS
// overrides it (at least 256) for tuning.  The MFMA kernel keeps this rule: with 32
// rows x 8 KV heads already in the grid, longer chunks measured slower (batched32,
// bf16 K/V: 118 us a step at 2048 blocks, 151 at 1024)
static int attn_batch_target() {
  static const int t = [] {
    const char* e = std::getenv("EAGLE3_ATTN_BATCH_BLOCKS");
    const int v = e ? std::atoi(e) : 0;
    return v >= 256 ? v : 2048;
  }();
  return t;
}

int attn_batch_chunk(const BatchRows& br, int m, int step, int n_head_kv, int head_dim, int kv_f32) {
  long long rows = 0;
  for (int r = 0; r < m; ++r) rows += br.row0[r] + step + 1;
  const int rpb = rows_per_block(head_dim, kv_f32);
  const long long target = attn_batch_target();
  long long c = (rows * n_head_kv + target - 1) / target;
  c = ((c + rpb - 1) / rpb) * rpb;
  if (c < kAttnBatchMinChunk) c = kAttnBatchMinChunk;
  if (c > kAttnMaxChunk) c = kAttnMaxChunk;
  return int(c);
}

int attn_batch_max_splits(int cap, int head_dim, int kv_f32) {
  (void)head_dim;
  (void)kv_f32;
  return (cap + kAttnBatchMinChunk - 1) / kAttnBatchMinChunk;
}

hipError_t launch_attn_batched(const AttnArgs& a, int m, uint16_t* out_hi, uint16_t* out_lo, int ld,
                               hipStream_t s) {
  if (!a.batched || m < 1 || m > kBatchRows) return hipErrorInvalidValue;
  const int chunk = attn_batch_chunk(a.br, m, a.step, a.n_head_kv, a.head_dim, a.kv_f32);
  int Tmax = 0;
  for (int r = 0; r < m; ++r) Tmax = std::max(Tmax, a.br.row0[r] + a.step + 1);
  const int Smax = (Tmax + chunk - 1) / chunk;
  if (Smax > attn_batch_max_splits(a.cap, a.head_dim, a.kv_f32) || Tmax > a.cap)
    return hipErrorInvalidValue;
  const int G = a.n_head / a.n_head_kv;
  hipError_t e = a.kv_f32 ? launch_kt<float>(a, G, chunk, Smax, s, m)
                          : launch_kt<uint16_t>(a, G, chunk, Smax, s, m);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine_b, dim3(a.n_head, m), dim3(128), size_t(Smax) * sizeof(float), s,
                     a.part_o, a.part_ml, Smax, a.head_dim, a.n_head, chunk, a.step, a.br, out_hi,
                     out_lo, ld);
  return hipGetLastError();
}

template <int HD>
static hipError_t launch_q_hd(const AttnArgs& a, int G, int chunk, int S, hipStream_t s) {
  dim3 grid(S, a.n_head_kv), block(64 * kAttnWaves);
#define E3_ATTN_CASE(GG)                                                      \
  case GG:                                                                  \
    hipLaunchKernelGGL((k_attn_q<HD, GG>), grid, block, 0, s, a, chunk, S); \
    break;
  switch (G) {
    E3_ATTN_CASE(1)
    E3_ATTN_CASE(2)
    E3_ATTN_CASE(3)
    E3_ATTN_CASE(4)
    E3_ATTN_CASE(5)
    E3_ATTN_CASE(6)
    E3_ATTN_CASE(7)
    E3_ATTN_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef E3_ATTN_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(a.n_head), dim3(HD), 0, s, a.part_o, a.part_ml, S, HD,
                     a.out);
  return hipGetLastError();
}

// query vectors per block of the verify attention: at most the decode kernel's
// largest G; 4 by default (at 32K rows, 40/8 heads and a 4-row window: 154 us fp32
// and 121 us bf16 against 160 and 161 with 8, whose 254 VGPRs leave 2 waves a SIMD)
constexpr int kVerifyGroup = 8;
constexpr int kVerifyGroupDefault = 4;

// EAGLE3_VERIFY_GROUP (1, 2, 4 or 8) caps it for tuning
static int verify_group(int MG) {
  static const int cap = [] {
    const char* e = std::getenv("EAGLE3_VERIFY_GROUP");
    const int v = e ? std::atoi(e) : 0;
    return (v == 1 || v == 2 || v == 4 || v == 8) ? v : kVerifyGroupDefault;
  }();
  const int g = MG <= 1 ? 1 : MG <= 2 ? 2 : MG <= 4 ? 4 : kVerifyGroup;
  return g < cap ? g : cap;
}

// EAGLE3_VERIFY_VALU=1 selects the VALU kernel (k_attn_mid) for comparison
static bool verify_valu() {
  static const bool v = [] {
    const char* e = std::getenv("EAGLE3_VERIFY_VALU");
    return e && e[0] == '1';
  }();
  return v;
}

// (KV head, split) tiles aimed at by the MFMA verify kernel (EAGLE3_VERIFY_BLOCKS
// overrides it): more than the decode kernel's, since a wave holds one 32-row tile's
// loads at a time
static int verify_blocks() {
  static const int t = [] {
    const char* e = std::getenv("EAGLE3_VERIFY_BLOCKS");
    const int v = e ? std::atoi(e) : 0;
    return (v >= 8 && v <= 8192) ? v : 1024;
  }();
  return t;
}

static bool verify_mfma(int hd) { return hd <= 128 && !verify_valu(); }

// EAGLE3_VERIFY_TILE32=1 selects the earlier MFMA kernel (32-row tiles, one in flight
// per wave) for comparison
static bool verify_tile32() {
  static const bool v = [] {
    const char* e = std::getenv("EAGLE3_VERIFY_TILE32");
    return e && e[0] == '1';
  }();
  return v;
}

static void verify_split(int T, int n_head_kv, int hd, int kv_f32, int* chunk, int* S) {
  if (verify_mfma(hd) && !verify_tile32()) pick_split_mfma(T, n_head_kv, chunk, S);
  else if (verify_mfma(hd)) pick_split(T, n_head_kv, hd, kv_f32, chunk, S, verify_blocks(), 32 * kAttnWaves);
  else pick_split(T, n_head_kv, hd, kv_f32, chunk, S);
}

size_t attn_verify_workspace(int M, int n_head, int n_head_kv, int head_dim, int ctx, int kv_f32) {
  int chunk, S;
  verify_split(ctx + M, n_head_kv, head_dim, kv_f32, &chunk, &S);
  return size_t(M) * n_head * S * (head_dim + 2) * sizeof(float);
}

template <int HD, typename KT>
static hipError_t launch_mid_hd(const VerifyArgs& a, int chunk, int S, hipStream_t s) {
  const int MG = a.M * (a.n_head / a.n_head_kv);
  // (head_dim 256 stays on the VALU kernel: the MFMA kernel's wave merge would need
  // more than 64 KB of LDS)
  if (verify_mfma(HD)) {
    const int QG = (MG + 15) / 16;
    const int tiles = S * a.n_head_kv;
    if (verify_tile32())
      hipLaunchKernelGGL((k_attn_mid_mfma<(HD <= 128 ? HD : 128), KT>), dim3(unsigned((tiles + 7) / 8 * 8 * QG)),
                         dim3(64 * kAttnWaves), 0, s, a, chunk, S, QG);
    else
      hipLaunchKernelGGL((k_attn_vr<(HD <= 128 ? HD : 128), KT>), dim3(unsigned((tiles + 7) / 8 * 8 * QG)),
                         dim3(64 * kAttnWaves), 0, s, a, chunk, S, QG);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3(a.M * a.n_head), dim3(HD), 0, s, a.part_o, a.part_ml, S,
                       HD, a.out);
    return hipGetLastError();
  }
  const int GQ = verify_group(MG);
  const int QG = (MG + GQ - 1) / GQ;
  const int tiles = S * a.n_head_kv;
  const dim3 grid(unsigned((tiles + 7) / 8 * 8 * QG)), block(64 * kAttnWaves);
  switch (GQ) {
    case 1: hipLaunchKernelGGL((k_attn_mid<HD, 1, KT>), grid, block, 0, s, a, chunk, S, QG); break;
    case 2: hipLaunchKernelGGL((k_attn_mid<HD, 2, KT>), grid, block, 0, s, a, chunk, S, QG); break;
    case 4: hipLaunchKernelGGL((k_attn_mid<HD, 4, KT>), grid, block, 0, s, a, chunk, S, QG); break;
    default: hipLaunchKernelGGL((k_attn_mid<HD, kVerifyGroup, KT>), grid, block, 0, s, a, chunk, S, QG); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(a.M * a.n_head), dim3(HD), 0, s, a.part_o, a.part_ml, S, HD,
                     a.out);
  return hipGetLastError();
}

hipError_t launch_attn_verify(const VerifyArgs& a, size_t workspace_bytes, hipStream_t s) {
  if (a.M < 1 || a.ctx < 0 || int64_t(a.ctx) + a.M > a.cap || a.n_head % a.n_head_kv)
    return hipErrorInvalidValue;
  int chunk, S;
  verify_split(a.ctx + a.M, a.n_head_kv, a.head_dim, a.kv_f32, &chunk, &S);
  if (S > 1 && workspace_bytes < attn_verify_workspace(a.M, a.n_head, a.n_head_kv, a.head_dim, a.ctx, a.kv_f32))
    return hipErrorInvalidValue;
  switch (a.head_dim) {
    case 64: return a.kv_f32 ? launch_mid_hd<64, float>(a, chunk, S, s) : launch_mid_hd<64, uint16_t>(a, chunk, S, s);
    case 128: return a.kv_f32 ? launch_mid_hd<128, float>(a, chunk, S, s) : launch_mid_hd<128, uint16_t>(a, chunk, S, s);
    case 256: return a.kv_f32 ? launch_mid_hd<256, float>(a, chunk, S, s) : launch_mid_hd<256, uint16_t>(a, chunk, S, s);
    default: return hipErrorInvalidValue;
  }
}


hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.batched) return hipErrorInvalidValue;
  // deferred QKV: fp32 or bf16 K/V, its register and LDS budgets (kDqPairs pairs per
  // thread, at most 16 query heads), and one batch of candidates per thread
  if (a.dq && (a.kv_q || !a.dq_hsum || !a.dqa.tok_tab || a.T < 1 ||
               (a.n_head / a.n_head_kv + 2) * (a.head_dim / 2) > kDqPairs * 64 * kAttnWaves ||
               a.n_head / a.n_head_kv > 16 || a.dqa.prev_count > kArgmaxBatch * 64 * kAttnWaves))
    return hipErrorInvalidValue;
  int chunk, S;
  const int G = a.n_head / a.n_head_kv;
  if (!a.kv_q && attn_on_mfma(a.head_dim, a.kv_f32, G)) pick_split_mfma(a.T, a.n_head_kv, &chunk, &S);
  else pick_split(a.T, a.n_head_kv, a.head_dim, a.kv_f32, &chunk, &S);
  if (a.kv_q) {
    if (a.head_dim <= 128 && G <= 16 && !attn_valu()) {
      // the MFMA kernel reads whole 16-row tiles: the region must hold a multiple of
      // 16 rows (zeroed at allocation)
      if (a.cap % 16) return hipErrorInvalidValue;
      // twice the blocks of the bf16 kernel: two waves a SIMD hide more of the
      // decode's latency (32767 rows, 40/8 heads: 40.7 us against 43.9 with 256,
      // attention and combine)
      pick_split_mfma(a.T, a.n_head_kv, &chunk, &S, std::getenv("EAGLE3_ATTN_BLOCKS") ? 0 : kAttnQmBlocks);
      // an odd number of 64-row wave steps per split: with an even number (512- or
      // 1024-row splits) every block's reads start at the same power-of-two offsets
      // and the kernel ran 25-40 % slower (32767 rows, 40/8 heads: 33-36 us against
      // 24-28 with 576-row splits)
      if (T_odd_steps() && (chunk / 64) % 2 == 0 && chunk < a.T) {
        chunk += 64;
        S = (a.T + chunk - 1) / chunk;
      }
      dim3 grid(S, a.n_head_kv), block(64 * kAttnWaves);
      if (qm_ring() == 4) {
        if (a.head_dim == 64) hipLaunchKernelGGL((k_attn_qm<64, 4>), grid, block, 0, s, a, chunk, S);
        else if (a.head_dim == 128) hipLaunchKernelGGL((k_attn_qm<128, 4>), grid, block, 0, s, a, chunk, S);
        else return hipErrorInvalidValue;
      } else if (a.head_dim == 64) hipLaunchKernelGGL((k_attn_qm<64, 3>), grid, block, 0, s, a, chunk, S);
      else if (a.head_dim == 128) hipLaunchKernelGGL((k_attn_qm<128, 3>), grid, block, 0, s, a, chunk, S);
      else return hipErrorInvalidValue;
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || S == 1) return e;
      hipLaunchKernelGGL(k_attn_combine, dim3(a.n_head), dim3(a.head_dim), 0, s, a.part_o, a.part_ml, S,
                         a.head_dim, a.out);
      return hipGetLastError();
    }
    switch (a.head_dim) {
      case 64: return launch_q_hd<64>(a, G, chunk, S, s);
      case 128: return launch_q_hd<128>(a, G, chunk, S, s);
      case 256: return launch_q_hd<256>(a, G, chunk, S, s);
      default: return hipErrorInvalidValue;
    }
  }
  return a.kv_f32 ? launch_kt<float>(a, G, chunk, S, s) : launch_kt<uint16_t>(a, G, chunk, S, s);
}

// ---------------------------------------------------------------------------
// Device-resident scratch of the allocation-free verify attention: the split
// partials of one call, at most kVerifyScratchBytes.  Every GPU the library runs
// on holds its own copy until the process ends; its device address is looked up
// once per device (with that device current) and kept.
}  // namespace e3

static __device__ __align__(256) unsigned char scratch[e3::kVerifyScratchBytes];

namespace e3 {

hipError_t verify_scratch_ptr(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *ptr = ptrs[dev];
  return hipSuccess;
}

}  // namespace e3
