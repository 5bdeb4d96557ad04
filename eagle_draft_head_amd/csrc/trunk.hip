// Kernels of the synthetic target trunk (a small Llama-style decoder) that checks
// the drafter's proposals: one forward over a window of T tokens appends T rows to
// the trunk's KV cache and gives every position's greedy token and its three tap
// features, and an accept walk compares a chain's drafts with those tokens.
//
// The trunk exists at test width (n_embd a few hundred), so these kernels are
// plain: every output element is computed by one thread (or one block) in a fixed
// order that does not depend on how many rows share the launch.  A row verified
// inside a window is therefore computed bit for bit as it would be alone, which is
// what makes greedy speculative decoding reproduce greedy decoding exactly.
// Attention over the trunk cache is the verify-window attention (attn.hip).
#include "common.hpp"
#include "kernels.hpp"

namespace e3 {

constexpr int kTrunkThreads = 256;

// x[t] = E[tok[t]] in fp32 (and a copy into the first tap); an id outside the
// vocabulary reads row 0 and raises bit 0 of the status word
__global__ __launch_bounds__(kTrunkThreads) void k_t_embed(const int32_t* __restrict__ tok,
                                                           const uint16_t* __restrict__ E, int n,
                                                           int vocab, float* __restrict__ x,
                                                           float* __restrict__ tap,
                                                           uint32_t* __restrict__ status) {
  const int t = blockIdx.x;
  int id = tok[t];
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) atomicOr(status, kTrunkBadToken);
    id = 0;
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float v = bf16_to_f32(E[(size_t)id * n + i]);
    x[(size_t)t * n + i] = v;
    if (tap) tap[(size_t)t * n + i] = v;
  }
}

// y[t] = w * x[t] / sqrt(mean(x[t]^2) + eps), one block per row
__global__ __launch_bounds__(kTrunkThreads) void k_t_rmsnorm(const float* __restrict__ x,
                                                             const float* __restrict__ w, int n,
                                                             float eps, float* __restrict__ y) {
  __shared__ float red[kTrunkThreads];
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * n;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ss = fmaf(xr[i], xr[i], ss);
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int o = kTrunkThreads / 2; o > 0; o >>= 1) {
    if (int(threadIdx.x) < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / float(n) + eps);
  for (int i = threadIdx.x; i < n; i += blockDim.x) y[(size_t)t * n + i] = w[i] * (xr[i] * inv);
}

// dot product of a bf16 row with an fp32 vector, K % 8 == 0, fixed order
__device__ __forceinline__ float t_dot(const uint16_t* __restrict__ w, const float* __restrict__ x, int K) {
  const uint4* w4 = reinterpret_cast<const uint4*>(w);
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float acc = 0.f;
  for (int c = 0; c < (K >> 3); ++c) acc = dot8(w4[c], x4[2 * c], x4[2 * c + 1], acc);
  return acc;
}

// Y[t][j] = W[j] . X[t] (+ R[t][j]); optionally also into Y2
__global__ __launch_bounds__(kTrunkThreads) void k_t_linear(const uint16_t* __restrict__ W, int N, int K,
                                                            const float* __restrict__ X,
                                                            const float* __restrict__ R,
                                                            float* __restrict__ Y, float* __restrict__ Y2) {
  const int t = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= N) return;
  float v = t_dot(W + (size_t)j * K, X + (size_t)t * K, K);
  if (R) v += R[(size_t)t * N + j];
  Y[(size_t)t * N + j] = v;
  if (Y2) Y2[(size_t)t * N + j] = v;
}

// act[t][i] = silu(Wg[i] . Z[t]) * (Wu[i] . Z[t])
__global__ __launch_bounds__(kTrunkThreads) void k_t_swiglu(const uint16_t* __restrict__ Wg,
                                                            const uint16_t* __restrict__ Wu, int ff,
                                                            int n, const float* __restrict__ Z,
                                                            float* __restrict__ act) {
  const int t = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ff) return;
  const float* z = Z + (size_t)t * n;
  const float g = t_dot(Wg + (size_t)i * n, z, n);
  const float u = t_dot(Wu + (size_t)i * n, z, n);
  act[(size_t)t * ff + i] = (g / (1.0f + expf(-g))) * u;
}

// NeoX rotation over the whole head (pairs (i, i + hd/2)) of row t's q and k heads
// at position pos0 + t; k and v rows go to cache rows pos0 + t ([nkv][cap][hd])
__global__ __launch_bounds__(kTrunkThreads) void k_t_rope_store(float* __restrict__ q,
                                                                const float* __restrict__ k,
                                                                const float* __restrict__ v, int nh,
                                                                int nkv, int hd, int pos0,
                                                                const double* __restrict__ inv_freq,
                                                                float* __restrict__ Kc,
                                                                float* __restrict__ Vc, int cap) {
  const int t = blockIdx.x;
  const int half = hd / 2, pos = pos0 + t;
  const int pairs = (nh + nkv) * half;
  for (int p = threadIdx.x; p < pairs; p += blockDim.x) {
    const int head = p / half, i = p - head * half;
    float c, s;
    rope_cs(pos, inv_freq[i], &c, &s);
    if (head < nh) {
      float* r = q + ((size_t)t * nh + head) * hd;
      const float a = r[i], b = r[i + half];
      r[i] = a * c - b * s;
      r[i + half] = b * c + a * s;
    } else {
      const int g = head - nh;
      const float* r = k + ((size_t)t * nkv + g) * hd;
      const float a = r[i], b = r[i + half];
      float* dst = Kc + ((size_t)g * cap + pos) * hd;
      dst[i] = a * c - b * s;
      dst[i + half] = b * c + a * s;
    }
  }
  for (int e = threadIdx.x; e < nkv * hd; e += blockDim.x) {
    const int g = e / hd, d = e - g * hd;
    Vc[((size_t)g * cap + pos) * hd + d] = v[(size_t)t * nkv * hd + e];
  }
}

// ids[t] = argmax logits[t] (the lowest index wins a tie; a NaN row raises bit 1 of
// the status word and gives id 0)
__global__ __launch_bounds__(kTrunkThreads) void k_t_argmax(const float* __restrict__ logits, int V,
                                                            int32_t* __restrict__ ids,
                                                            uint32_t* __restrict__ status) {
  __shared__ float sv[kTrunkThreads / kWave];
  __shared__ int si[kTrunkThreads / kWave];
  const int t = blockIdx.x;
  const float* r = logits + (size_t)t * V;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x; i < V; i += blockDim.x)
    if (better(r[i], i, bv, bi)) { bv = r[i]; bi = i; }
  wave_argmax(bv, bi);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < int(blockDim.x >> 6); ++k)
      if (better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
    if (bi < 0 || bi >= V) {  // every logit NaN
      atomicOr(status, kTrunkNanLogits);
      bi = 0;
    }
    ids[t] = bi;
  }
}

// The accept walk of greedy verification: a = the longest prefix with
// drafts[i] == verify[i] (i < g), bonus = verify[a].  res = [a, bonus, status,
// drafts...]; the status word is handed over and cleared.
__global__ void k_accept(const int32_t* __restrict__ drafts, const int32_t* __restrict__ verify, int g,
                         int32_t* __restrict__ res, uint32_t* __restrict__ status) {
  if (threadIdx.x != 0) return;
  int a = 0;
  while (a < g && drafts[a] == verify[a]) ++a;
  res[0] = a;
  res[1] = verify[a];
  res[2] = int32_t(*status);
  *status = 0u;
  for (int i = 0; i < g; ++i) res[3 + i] = drafts[i];
}

static dim3 rows_grid(int N, int T) { return dim3(unsigned((N + kTrunkThreads - 1) / kTrunkThreads), unsigned(T)); }

hipError_t launch_trunk_forward(const TrunkArgs& a, int T, int pos0, const int32_t* tok, int32_t* ids,
                                float* const taps[3], hipStream_t s) {
  const int n = a.n, qd = a.nh * a.hd, kvd = a.nkv * a.hd;
  const TrunkBufs& b = a.buf;
  hipLaunchKernelGGL(k_t_embed, dim3(T), dim3(kTrunkThreads), 0, s, tok, a.embed, n, a.vocab, b.x,
                     taps[0], a.status);
  for (int l = 0; l < a.n_layers; ++l) {
    const TrunkLayer& L = a.layer[l];
    hipLaunchKernelGGL(k_t_rmsnorm, dim3(T), dim3(kTrunkThreads), 0, s, b.x, L.attn_norm, n, a.eps, b.z);
    hipLaunchKernelGGL(k_t_linear, rows_grid(qd, T), dim3(kTrunkThreads), 0, s, L.wq, qd, n, b.z,
                       nullptr, b.q, nullptr);
    hipLaunchKernelGGL(k_t_linear, rows_grid(kvd, T), dim3(kTrunkThreads), 0, s, L.wk, kvd, n, b.z,
                       nullptr, b.k, nullptr);
    hipLaunchKernelGGL(k_t_linear, rows_grid(kvd, T), dim3(kTrunkThreads), 0, s, L.wv, kvd, n, b.z,
                       nullptr, b.v, nullptr);
    hipLaunchKernelGGL(k_t_rope_store, dim3(T), dim3(kTrunkThreads), 0, s, b.q, b.k, b.v, a.nh, a.nkv,
                       a.hd, pos0, a.inv_freq, L.k_cache, L.v_cache, a.cap);
    VerifyArgs va{};
    va.q = b.q; va.k = L.k_cache; va.v = L.v_cache; va.kv_f32 = 1;
    va.cap = a.cap; va.ctx = pos0; va.M = T;
    va.n_head = a.nh; va.n_head_kv = a.nkv; va.head_dim = a.hd;
    va.part_o = b.part_o; va.part_ml = b.part_ml; va.out = b.o;
    hipError_t e = launch_attn_verify(va, b.ws_bytes, s);
    if (e != hipSuccess) return e;
    // h = x + o_proj(o); the MLP input z = RMSNorm(h); x = h + down(silu(gate z) * up z)
    hipLaunchKernelGGL(k_t_linear, rows_grid(n, T), dim3(kTrunkThreads), 0, s, L.wo, n, qd, b.o, b.x,
                       b.h, nullptr);
    hipLaunchKernelGGL(k_t_rmsnorm, dim3(T), dim3(kTrunkThreads), 0, s, b.h, L.mlp_norm, n, a.eps, b.z);
    hipLaunchKernelGGL(k_t_swiglu, rows_grid(a.ff, T), dim3(kTrunkThreads), 0, s, L.w_gate, L.w_up,
                       a.ff, n, b.z, b.act);
    float* tap = (l + 1 == a.n_layers / 2) ? taps[1] : (l + 1 == a.n_layers ? taps[2] : nullptr);
    hipLaunchKernelGGL(k_t_linear, rows_grid(n, T), dim3(kTrunkThreads), 0, s, L.w_down, n, a.ff, b.act,
                       b.h, b.x, tap);
  }
  hipLaunchKernelGGL(k_t_rmsnorm, dim3(T), dim3(kTrunkThreads), 0, s, b.x, a.final_norm, n, a.eps, b.z);
  hipLaunchKernelGGL(k_t_linear, rows_grid(a.vocab, T), dim3(kTrunkThreads), 0, s, a.lm_head, a.vocab, n,
                     b.z, nullptr, b.logits, nullptr);
  hipLaunchKernelGGL(k_t_argmax, dim3(T), dim3(kTrunkThreads), 0, s, b.logits, a.vocab, ids, a.status);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* drafts, const int32_t* verify, int g, int32_t* res,
                         uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(64), 0, s, drafts, verify, g, res, status);
  return hipGetLastError();
}

}  // namespace e3
