// GEMV family: y = W x with bf16 weights streamed from HBM in 16-byte
// coalesced loads and fp32 activations staged in LDS, fp32 accumulate.
//
// RMSNorm is split between producer and consumer: a kernel whose output y
// feeds a norm also writes y * w_norm (the consumer's weight) and one partial
// sum of y^2 per block; the consumer stages the weighted vector as is, adds the
// partial sums and applies 1/rms in its epilogue.  So no prologue loads norm
// weights or reduces before streaming.
//   k_encode      g = fc . [taps]            -> g, g*w_hid, partial sum g^2
//   k_qkv         [finish the previous step's argmax + d2t] -> token; streams the
//                 hidden half of W_qkv first while the token's embedding row is
//                 in flight, then the embedding half; epilogue: 1/rms per half,
//                 NeoX rotation (q/k rows repacked so partners are adjacent),
//                 q to fp32, k/v rows to the KV cache
//   k_qkv_tab     k_qkv with the token table: the embedding half is one table row,
//                 only the hidden half streams (from its own contiguous copy)
//   k_gemv_resid  y = W x + resid            -> y, y*w1, y*w2, partial sum y^2
//   k_gateup      silu(gate . z) * (up . z) with z = x1*w_post/rms (rows interleaved)
//   k_lmhead      logits = lm_head . (h*w_norm/rms) -> per-block (max, argmax)
//   k_lmhead_qh   k_lmhead plus the next step's hidden-half QKV sums (deferred
//                 QKV: the attention kernel finishes that step's q and K/V row)
// The multi-vector kernel (teacher-forced rows) applies each weight chunk to
// M activation vectors and splits K so the M vectors fit in LDS (with int4 weights
// as five-digit fixed point per group, v_dot8 products); it writes split partials
// that the next kernel sums.  k_gemv_multi_qh is its K/V pass
// with the hidden-half QKV sums of the boundary feature the pass writes in the
// same launch (the next chain's first step then starts at its attention).
//
// Work split: a wave owns R consecutive rows; lane l reads 16-byte chunks
// l, l+64, ... of each row (1 KB per row per wave instruction); U chunk steps
// are issued before their FMAs so each lane keeps U*R loads in flight.  The
// per-row sums are reduced across the wave at the end.  No block ever waits
// for another block: cross-block reductions happen in the next kernel.
#include <algorithm>
#include <cstdlib>

#include <hip/hip_ext.h>

#include "common.hpp"
#include "gemv_cfg.hpp"
#include "kernels.hpp"
#include "qkv_token.hpp"

namespace e3 {

// hipLaunchKernelGGL, or the event-timed extended launch when armed (LaunchEvents)
#define E3_LAUNCH(K, G, B, SH, S, ...)                                                         \
  do {                                                                                         \
    if (g_launch_ev.armed)                                                                     \
      hipExtLaunchKernelGGL(K, G, B, SH, S, g_launch_ev.start, g_launch_ev.stop, 0, __VA_ARGS__); \
    else                                                                                       \
      hipLaunchKernelGGL(K, G, B, SH, S, __VA_ARGS__);                                          \
  } while (0)


// Row pointers of the R rows a wave owns, at column k0 (rows past N repeat the last row).
template <int R>
__device__ __forceinline__ void row_ptrs(const uint16_t* __restrict__ W, size_t ldw, int row0, int N,
                                         int k0, const uint4* (&wp)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
    wp[r] = reinterpret_cast<const uint4*>(W + (size_t)min(row0 + r, N - 1) * ldw + k0);
}

// Continue the dot products from 16-byte chunk c (this lane's) to the end: U chunk
// steps in flight per row, then single steps for the tail.
template <int R, int U>
__device__ __forceinline__ void rows_dot_from(const uint4* (&wp)[R], int c, int nch,
                                              const float4* __restrict__ x4, float (&acc)[R]) {
  for (; c + 64 * (U - 1) < nch; c += 64 * U) {
    uint4 w[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) w[u][r] = ld_stream(wp[r] + c + 64 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float4 a = x4[2 * (c + 64 * u)], b = x4[2 * (c + 64 * u) + 1];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = dot8(w[u][r], a, b, acc[r]);
    }
  }
  for (; c < nch; c += 64) {
    uint4 t[R];
#pragma unroll
    for (int r = 0; r < R; ++r) t[r] = ld_stream(wp[r] + c);
    const float4 a = x4[2 * c], b = x4[2 * c + 1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = dot8(t[r], a, b, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
}

// Stream columns [k0, k0 + K) of the R rows a wave owns against xs[0, K).
template <int R, int U>
__device__ __forceinline__ void rows_dot(const uint16_t* __restrict__ W, size_t ldw, int row0,
                                         int N, int k0, int K, const float* __restrict__ xs,
                                         float (&acc)[R]) {
  const uint4* wp[R];
  row_ptrs<R>(W, ldw, row0, N, k0, wp);
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  rows_dot_from<R, U>(wp, threadIdx.x & 63, K >> 3, reinterpret_cast<const float4*>(xs), acc);
}

// The first U chunk steps of rows_dot, issued early (before a prologue whose
// loads can then complete behind them); requires K / 8 >= 64 U.
template <int R, int U>
__device__ __forceinline__ void rows_issue(const uint16_t* __restrict__ W, size_t ldw, int row0,
                                           int N, int k0, uint4 (&w)[U][R]) {
  const uint4* wp[R];
  row_ptrs<R>(W, ldw, row0, N, k0, wp);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) w[u][r] = ld_stream(wp[r] + lane + 64 * u);
}

// rows_dot whose first U chunk steps were issued by rows_issue.
template <int R, int U>
__device__ __forceinline__ void rows_dot_issued(const uint16_t* __restrict__ W, size_t ldw, int row0,
                                                int N, int k0, int K, const float* __restrict__ xs,
                                                const uint4 (&w)[U][R], float (&acc)[R]) {
  const uint4* wp[R];
  row_ptrs<R>(W, ldw, row0, N, k0, wp);
  const int lane = threadIdx.x & 63;
  const float4* x4 = reinterpret_cast<const float4*>(xs);
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float4 a = x4[2 * (lane + 64 * u)], b = x4[2 * (lane + 64 * u) + 1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = dot8(w[u][r], a, b, acc[r]);
  }
  rows_dot_from<R, U>(wp, lane + 64 * U, K >> 3, x4, acc);
}

// ---------------------------------------------------------------------------
// int4 weights (kernels.hpp, I4 weights): a row of K weights is K / 2 bytes of
// codes (element 2i in the low nibble, stored as q + 8) and K / 32 bf16 scales, one
// per group of 32.  A lane's 16-byte chunk is one whole group.
//
// The activation vector is turned once per block into fixed point per group of 32:
// a power-of-two exponent e from the group's largest magnitude m (2^(E-1) <= m < 2^E,
// e = 14 - E) and x_q = rint(x * 2^e), so |x_q| <= 2^14 and x_q is off from x * 2^e
// by at most 1/2, i.e. x by at most m * 2^-14.  x_q + 0x8888 has four base-16
// digits u_t, and x_q = sum_t 16^t (u_t - 8); the digits (u_t - 8) are stored as
// signed nibbles, one plane per t, in the element order of the codes.  A code XOR 8
// is q as a signed nibble, so sixteen v_dot8_i32_i4 give the four per-digit sums of
// a group exactly, and sum_t 16^t s_t = sum q x_q (|.| < 2^22, exact in fp32) is
// scaled by scale * 2^-e once per group and row.

// LDS layout of a vector of G groups: planes [4][G] uint4 (entry i * G + g holds
// digit planes 0..3 of elements 8i..8i+7 of group g) and exponents [G] int.
constexpr size_t q_vec_bytes(int K) { return size_t(K / 8) * 16 + size_t(K / 32) * 4; }

// swap nibbles 1 <-> 2 and 5 <-> 6 of a word
__device__ __forceinline__ uint32_t swap_mid_nibbles(uint32_t x) {
  const uint32_t t = ((x >> 4) ^ x) & 0x00F000F0u;
  return x ^ t ^ (t << 4);
}

// xs[0, K) (fp32, LDS) -> digit planes xp and exponents xe (LDS).  Every thread of
// the block calls it; K % 32 == 0 and blockDim.x % 64 == 0.  One thread per 8
// elements; the four threads of a group are the four lanes of a DPP quad.
__device__ __forceinline__ void quant_x_i4(const float* __restrict__ xs, int K,
                                           uint4* __restrict__ xp, int* __restrict__ xe) {
  const int G = K >> 5, nchunk = K >> 3;
  const float4* x4 = reinterpret_cast<const float4*>(xs);
  for (int j0 = 0; j0 < nchunk; j0 += blockDim.x) {  // same trip count for every lane
    const int j = j0 + int(threadIdx.x);
    const bool on = j < nchunk;  // whole quads are on or off (nchunk % 4 == 0)
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (on) {
      a = x4[2 * j];
      b = x4[2 * j + 1];
    }
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
    m = fmaxf(m, dpp_move<kDppQuadSwap1>(m));
    m = fmaxf(m, dpp_move<kDppQuadSwap2>(m));
    const int e = 14 - (int((__float_as_uint(m) >> 23) & 0xFFu) - 126);
    uint32_t u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float t = __builtin_amdgcn_fmed3f(rintf(ldexpf(v[k], e)), -16384.f, 16384.f);
      u[k] = uint32_t(int(t) + 0x8888);  // 16 bits
    }
    // d_i: byte t = digit t of element 2i (low nibble) and of element 2i + 1 (high)
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = swap_mid_nibbles(__builtin_amdgcn_perm(u[2 * i + 1], u[2 * i], 0x05010400u));
    // byte transpose: plane t = byte t of d_0..d_3
    const uint32_t t01l = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);
    const uint32_t t01h = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);
    const uint32_t t23l = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
    const uint32_t t23h = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
    const uint4 pl = make_uint4(__builtin_amdgcn_perm(t23l, t01l, 0x05040100u) ^ 0x88888888u,
                                __builtin_amdgcn_perm(t23l, t01l, 0x07060302u) ^ 0x88888888u,
                                __builtin_amdgcn_perm(t23h, t01h, 0x05040100u) ^ 0x88888888u,
                                __builtin_amdgcn_perm(t23h, t01h, 0x07060302u) ^ 0x88888888u);
    if (on) {
      xp[(j & 3) * G + (j >> 2)] = pl;
      if ((j & 3) == 0) xe[j >> 2] = e;
    }
  }
}

// The five-digit form for the teacher-forced rows (their K/V rows are stored, so they
// keep about the precision of fp32 products): e = 18 - E, |x_q| <= 2^18, and
// x_q + 0x88888 has five base-16 digits; planes 0..3 laid out as above, plane 4 as
// [G] uint4 (component i holds elements 8i..8i+7 of group g).
// Eight elements of a group (one of its four quads of threads) in five-digit fixed
// point: planes 0..3 (pl), plane 4 (p4, element k in nibble k) and the group's
// exponent e.  Every lane of the quad calls it (the group maximum is a quad reduction).
__device__ __forceinline__ void quant8_5(const float (&v)[8], uint4& pl, uint32_t& p4, int& e) {
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  m = fmaxf(m, dpp_move<kDppQuadSwap1>(m));
  m = fmaxf(m, dpp_move<kDppQuadSwap2>(m));
  e = 18 - (int((__float_as_uint(m) >> 23) & 0xFFu) - 126);
  uint32_t u[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float t = __builtin_amdgcn_fmed3f(rintf(ldexpf(v[k], e)), -262144.f, 262144.f);
    u[k] = uint32_t(int(t) + 0x88888);  // 20 bits
  }
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = swap_mid_nibbles(__builtin_amdgcn_perm(u[2 * i + 1], u[2 * i], 0x05010400u));
  const uint32_t t01l = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);
  const uint32_t t01h = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);
  const uint32_t t23l = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
  const uint32_t t23h = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
  pl = make_uint4(__builtin_amdgcn_perm(t23l, t01l, 0x05040100u) ^ 0x88888888u,
                  __builtin_amdgcn_perm(t23l, t01l, 0x07060302u) ^ 0x88888888u,
                  __builtin_amdgcn_perm(t23h, t01h, 0x05040100u) ^ 0x88888888u,
                  __builtin_amdgcn_perm(t23h, t01h, 0x07060302u) ^ 0x88888888u);
  uint32_t q = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) q |= ((u[k] >> 16) & 0xFu) << (4 * k);
  p4 = q ^ 0x88888888u;
}

// q_group with the five digit planes
template <int R>
__device__ __forceinline__ void q_group5(const uint4 (&w)[R], const uint16_t (&sc)[R], int g, int G,
                                         const uint4* __restrict__ xp, const uint4* __restrict__ x4p,
                                         const int* __restrict__ xe, float (&acc)[R]) {
  const uint4 p0 = xp[g], p1 = xp[G + g], p2 = xp[2 * G + g], p3 = xp[3 * G + g], p4 = x4p[g];
  const int e = xe[g];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int w0 = int(w[r].x ^ 0x88888888u), w1 = int(w[r].y ^ 0x88888888u);
    const int w2 = int(w[r].z ^ 0x88888888u), w3 = int(w[r].w ^ 0x88888888u);
    const uint32_t pp[5][4] = {{p0.x, p1.x, p2.x, p3.x}, {p0.y, p1.y, p2.y, p3.y}, {p0.z, p1.z, p2.z, p3.z},
                               {p0.w, p1.w, p2.w, p3.w}, {p4.x, p4.y, p4.z, p4.w}};
    int gs = 0;
#pragma unroll
    for (int t = 4; t >= 0; --t) {
      if (t < 4) gs <<= 4;
      gs = __builtin_amdgcn_sdot8(w0, int(pp[t][0]), gs, false);
      gs = __builtin_amdgcn_sdot8(w1, int(pp[t][1]), gs, false);
      gs = __builtin_amdgcn_sdot8(w2, int(pp[t][2]), gs, false);
      gs = __builtin_amdgcn_sdot8(w3, int(pp[t][3]), gs, false);
    }
    acc[r] = fmaf(ldexpf(float(gs), -e), bf16_to_f32(sc[r]), acc[r]);
  }
}

// group g of the lane (of G in the vector) applied to the R rows
template <int R>
__device__ __forceinline__ void q_group(const uint4 (&w)[R], const uint16_t (&sc)[R], int g, int G,
                                        const uint4* __restrict__ xp, const int* __restrict__ xe,
                                        float (&acc)[R]) {
  const uint4 p0 = xp[g], p1 = xp[G + g], p2 = xp[2 * G + g], p3 = xp[3 * G + g];
  const int e = xe[g];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int w0 = int(w[r].x ^ 0x88888888u), w1 = int(w[r].y ^ 0x88888888u);
    const int w2 = int(w[r].z ^ 0x88888888u), w3 = int(w[r].w ^ 0x88888888u);
    const uint32_t pp[4][4] = {{p0.x, p1.x, p2.x, p3.x}, {p0.y, p1.y, p2.y, p3.y},
                               {p0.z, p1.z, p2.z, p3.z}, {p0.w, p1.w, p2.w, p3.w}};
    // Horner over the digit planes, most significant first: one chain of 16 dots
    int gs = 0;
#pragma unroll
    for (int t = 3; t >= 0; --t) {
      if (t < 3) gs <<= 4;
      gs = __builtin_amdgcn_sdot8(w0, int(pp[t][0]), gs, false);
      gs = __builtin_amdgcn_sdot8(w1, int(pp[t][1]), gs, false);
      gs = __builtin_amdgcn_sdot8(w2, int(pp[t][2]), gs, false);
      gs = __builtin_amdgcn_sdot8(w3, int(pp[t][3]), gs, false);
    }
    acc[r] = fmaf(ldexpf(float(gs), -e), bf16_to_f32(sc[r]), acc[r]);
  }
}

// The first U chunk steps (codes and scales) of the R int4 rows a wave owns, from
// codes Q and scales S of a matrix of row length ldw, columns [k0, k0 + K) (k0 and
// K multiples of 32): issued before the prologue that stages the vector, so that
// the weight stream overlaps it.
template <int R, int U>
struct QLoad {
  uint4 w[U][R];
  uint16_t sc[U][R];
};

template <int R>
__device__ __forceinline__ void q_row_ptrs(const uint8_t* __restrict__ Q, const uint16_t* __restrict__ S,
                                           size_t ldw, int row0, int N, int k0,
                                           const uint4* (&wp)[R], const uint16_t* (&sp)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = (size_t)min(row0 + r, N - 1);
    wp[r] = reinterpret_cast<const uint4*>(Q + row * (ldw / 2) + k0 / 2);
    sp[r] = S + row * (ldw / 32) + k0 / 32;
  }
}

template <int R, int U>
__device__ __forceinline__ void q_issue(const uint8_t* __restrict__ Q, const uint16_t* __restrict__ S,
                                        size_t ldw, int row0, int N, int k0, int K, QLoad<R, U>& L) {
  const uint4* wp[R];
  const uint16_t* sp[R];
  q_row_ptrs<R>(Q, S, ldw, row0, N, k0, wp, sp);
  const int G = K >> 5, lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    if (c < G) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        L.w[u][r] = ld_stream(wp[r] + c);
        L.sc[u][r] = sp[r][c];
      }
    }
  }
}

// the dot products of those rows against the quantised vector (xp, xe) of the K
// columns: the issued steps, then the rest of the row one step at a time
template <int R, int U>
__device__ __forceinline__ void q_dot_issued(const uint8_t* __restrict__ Q,
                                             const uint16_t* __restrict__ S, size_t ldw, int row0,
                                             int N, int k0, int K, const QLoad<R, U>& L,
                                             const uint4* __restrict__ xp, const int* __restrict__ xe,
                                             float (&acc)[R]) {
  const int G = K >> 5, lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (lane + 64 * u < G) q_group<R>(L.w[u], L.sc[u], lane + 64 * u, G, xp, xe, acc);
  if (64 * U < G) {
    const uint4* wp[R];
    const uint16_t* sp[R];
    q_row_ptrs<R>(Q, S, ldw, row0, N, k0, wp, sp);
    for (int c = lane + 64 * U; c < G; c += 64) {
      uint4 w[R];
      uint16_t sc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[r] = ld_stream(wp[r] + c);
        sc[r] = sp[r][c];
      }
      q_group<R>(w, sc, c, G, xp, xe, acc);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
}

// int4 kernels keep 4 waves per SIMD resident (at most 128 VGPRs): a wave's loads
// are one row set's worth, so the loads of other waves hide its arithmetic
constexpr int kI4WavesPerSimd = 4;

// int4 kernels run a grid of at most this many blocks (each stages and quantises
// the vector once, then covers ceil(virtual blocks / grid) virtual blocks of rows);
// EAGLE3_I4_BLOCKS overrides it
constexpr int kI4Blocks = 512;
int i4_blocks() {
  static const int v = [] {
    const char* s = std::getenv("EAGLE3_I4_BLOCKS");
    const int b = s ? std::atoi(s) : 0;
    return b > 0 ? b : kI4Blocks;
  }();
  return v;
}
// the launched grid for nvb virtual blocks: the fewest blocks that keep the
// per-block count of virtual blocks at ceil(nvb / cap)
static inline int i4_grid(int nvb) {
  const int cap = i4_blocks();
  if (nvb <= cap) return nvb;
  const int per = (nvb + cap - 1) / cap;
  return (nvb + per - 1) / per;
}

// One thread per group of 32: scale = bf16(max|w| / 7), codes rint(w / scale)
// clamped to [-7, 7] (both divisions IEEE fp32), stored as nibbles q + 8.
__global__ __launch_bounds__(256) void k_quant_i4(const uint16_t* __restrict__ W, int rows, int K,
                                                  uint8_t* __restrict__ Q, uint16_t* __restrict__ S) {
  const int gpr = K >> 5;
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (size_t)rows * gpr) return;
  const size_t row = g / gpr, gi = g - row * gpr;
  const uint4* src = reinterpret_cast<const uint4*>(W + row * K + gi * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    v[8 * i + 0] = bf16_lo(u.x); v[8 * i + 1] = bf16_hi(u.x);
    v[8 * i + 2] = bf16_lo(u.y); v[8 * i + 3] = bf16_hi(u.y);
    v[8 * i + 4] = bf16_lo(u.z); v[8 * i + 5] = bf16_hi(u.z);
    v[8 * i + 6] = bf16_lo(u.w); v[8 * i + 7] = bf16_hi(u.w);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint16_t sb = f32_to_bf16(__fdiv_rn(amax, 7.0f));
  const float sc = bf16_to_f32(sb);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int q = 0;
    if (sc > 0.f) q = (int)fminf(fmaxf(rintf(__fdiv_rn(v[i], sc)), -7.f), 7.f);
    words[i >> 3] |= uint32_t(q + 8) << (4 * (i & 7));
  }
  *reinterpret_cast<uint4*>(Q + row * (K / 2) + gi * 16) = make_uint4(words[0], words[1], words[2], words[3]);
  S[row * gpr + gi] = sb;
}

// One thread per weight: w = scale * q (at most 11 significant bits) as bf16 hi (round
// to nearest even) and lo = w - hi, which is exact in bf16, so hi + lo == w.
__global__ __launch_bounds__(256) void k_dequant_i4_split(const uint8_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ S, int rows,
                                                          int K, uint16_t* __restrict__ hi,
                                                          uint16_t* __restrict__ lo) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * K) return;
  const size_t row = i / K, k = i - row * K;
  const uint8_t b = Q[row * (K / 2) + k / 2];
  const int q = int((k & 1) ? (b >> 4) : (b & 15)) - 8;
  const float w = bf16_to_f32(S[row * (K / 32) + k / 32]) * float(q);
  const uint16_t h = f32_to_bf16(w);
  hi[i] = h;
  lo[i] = f32_to_bf16(w - bf16_to_f32(h));
}

hipError_t launch_dequant_i4_split(const uint8_t* Q, const uint16_t* S, int rows, int K, uint16_t* hi,
                                   uint16_t* lo, hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K % 32)) return hipErrorInvalidValue;
  const size_t n = (size_t)rows * K;
  hipLaunchKernelGGL(k_dequant_i4_split, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, Q, S, rows, K,
                     hi, lo);
  return hipGetLastError();
}

hipError_t launch_quant_i4(const uint16_t* W, int rows, int K, uint8_t* Q, uint16_t* S, hipStream_t s) {
  if (rows <= 0 || K <= 0 || (K % 32)) return hipErrorInvalidValue;
  const size_t groups = (size_t)rows * (K / 32);
  hipLaunchKernelGGL(k_quant_i4, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s, W, rows, K, Q, S);
  return hipGetLastError();
}


// Emit the R rows of a wave: y, y*w1, y*w2 (when given) and the block's sum of
// y^2 (when given) as partial `slot`.  Every thread of the block must call it.
template <int R, int WAVES>
__device__ __forceinline__ void emit_rows(const float (&y)[R], int row0, int N, const VecOut& o,
                                          float* red, int slot) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    if (row < N) {
      if (lane == r) {
        o.y[row] = y[r];
        if (o.yw1) o.yw1[row] = y[r] * o.w1[row];
        if (o.yw2) o.yw2[row] = y[r] * o.w2[row];
      }
      ss = fmaf(y[r], y[r], ss);
    }
  }
  if (!o.ssq) return;
  if (lane == 0) red[wv] = ss;  // every lane holds the same y[] after the reduction
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[w];
    o.ssq[slot] = t;
  }
}

// xs[i] = e[i] * w[i] for a bf16 row e; returns the share of sum(e^2)
__device__ __forceinline__ float stage_weighted_bf16(float* xs, const uint16_t* __restrict__ e,
                                                     const float* __restrict__ w, int n) {
  const uint2* e4 = reinterpret_cast<const uint2*>(e);
  const float4* w4 = reinterpret_cast<const float4*>(w);
  float4* x4 = reinterpret_cast<float4*>(xs);
  float ss = 0.f;
#pragma unroll 4
  for (int i = threadIdx.x; i < (n >> 2); i += blockDim.x) {
    const uint2 u = e4[i];
    const float4 b = w4[i];
    const float a0 = bf16_lo(u.x), a1 = bf16_hi(u.x), a2 = bf16_lo(u.y), a3 = bf16_hi(u.y);
    x4[i] = make_float4(a0 * b.x, a1 * b.y, a2 * b.z, a3 * b.w);
    ss = fmaf(a0, a0, fmaf(a1, a1, fmaf(a2, a2, fmaf(a3, a3, ss))));
  }
  return ss;
}

// xs[0:n) = v  (n % 4 == 0)
__device__ __forceinline__ void stage_plain(float* xs, const float* __restrict__ v, int n) {
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float4* x4 = reinterpret_cast<float4*>(xs);
#pragma unroll 4
  for (int i = threadIdx.x; i < (n >> 2); i += blockDim.x) x4[i] = v4[i];
}


// ---------------------------------------------------------------------------
template <int WAVES, int R, int U, bool I4>
__global__ __launch_bounds__(64 * WAVES, I4 ? kI4WavesPerSimd : 1) void k_encode(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ S, int n,
    const float* __restrict__ a0, const float* __restrict__ a1, const float* __restrict__ a2,
    VecOut out) {
  extern __shared__ float xs[];  // [3n]; int4: then the quantised vector
  __shared__ float red[16];
  const int wv = threadIdx.x >> 6;
  if constexpr (!I4) {
    stage_plain(xs, a0, n);
    stage_plain(xs + n, a1, n);
    stage_plain(xs + 2 * n, a2, n);
    __syncthreads();
    const int row0 = (blockIdx.x * WAVES + wv) * R;
    float acc[R];
    if (row0 < n) rows_dot<R, U>(W, size_t(3) * n, row0, n, 0, 3 * n, xs, acc);
    else
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
    emit_rows<R, WAVES>(acc, row0, n, out, red, blockIdx.x);
  } else {
    const uint8_t* Q = reinterpret_cast<const uint8_t*>(W);
    const int K = 3 * n;
    const int nvb = (n + WAVES * R - 1) / (WAVES * R);
    QLoad<R, U> L;
    int row0 = (blockIdx.x * WAVES + wv) * R;
    if (row0 < n) q_issue<R, U>(Q, S, size_t(K), row0, n, 0, K, L);
    stage_plain(xs, a0, n);
    stage_plain(xs + n, a1, n);
    stage_plain(xs + 2 * n, a2, n);
    __syncthreads();
    uint4* xp = reinterpret_cast<uint4*>(xs + K);
    int* xe = reinterpret_cast<int*>(xp + K / 8);
    quant_x_i4(xs, K, xp, xe);
    __syncthreads();
    // (the whole row is one issue for the drafter widths and the grid covers every
    // row set, so the loop body runs once; later row sets load at their turn)
    for (int vb = blockIdx.x;; vb += gridDim.x) {
      float acc[R];
      if (row0 < n) q_dot_issued<R, U>(Q, S, size_t(K), row0, n, 0, K, L, xp, xe, acc);
      else
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
      emit_rows<R, WAVES>(acc, row0, n, out, red, vb);
      const int vn = vb + int(gridDim.x);
      if (vn >= nvb) break;
      __syncthreads();  // red is reused by the next virtual block
      row0 = (vn * WAVES + wv) * R;
      if (row0 < n) q_issue<R, U>(Q, S, size_t(K), row0, n, 0, K, L);
    }
  }
}

// ---------------------------------------------------------------------------
constexpr int kQkvERegs = 8;  // float4 chunks of the embedding row held per thread

// the fused epilogue of a wave's R rows: 1/rms per half, NeoX rotation of q/k
// pairs, q to fp32, k/v rows to the KV cache
template <int R>
__device__ __forceinline__ void qkv_epilogue(const QkvArgs& a, int row0, const float (&acc_e)[R],
                                             const float (&acc_g)[R], float ie, float ig) {
  const int lane = threadIdx.x & 63;
  const int hd = a.head_dim;
  const int qd = a.n_head * hd, kvd = a.n_head_kv * hd;
  const int N = qd + 2 * kvd;
#pragma unroll
  for (int p = 0; p < R / 2; ++p) {
    const int r = row0 + 2 * p;
    if (lane != p || r >= N) continue;
    float y0 = acc_e[2 * p] * ie + acc_g[2 * p] * ig;
    float y1 = acc_e[2 * p + 1] * ie + acc_g[2 * p + 1] * ig;
    int seg, rr;
    if (r < qd) { seg = 0; rr = r; }
    else if (r < qd + kvd) { seg = 1; rr = r - qd; }
    else { seg = 2; rr = r - qd - kvd; }
    const int head = rr / hd, li = rr - head * hd;
    int d0 = li, d1 = li + 1;
    if (seg < 2 && li < a.rope_dim) {
      const int i = li >> 1;
      d0 = i;
      d1 = i + (a.rope_dim >> 1);
      float c, s;
      rope_cs(a.pos, a.inv_freq[i], &c, &s);
      const float t0 = y0 * c - y1 * s;
      const float t1 = y1 * c + y0 * s;
      y0 = t0;
      y1 = t1;
    }
    if (seg == 0) {
      a.q_out[head * hd + d0] = y0;
      a.q_out[head * hd + d1] = y1;
    } else {
      void* base = seg == 1 ? a.k_cache : a.v_cache;
      const size_t row = ((size_t)head * a.cap + a.row) * hd;
      kv_store(base, row + d0, y0, a.kv_f32);
      kv_store(base, row + d1, y1, a.kv_f32);
    }
  }
}

template <int WAVES, int R, int U>
__global__ __launch_bounds__(64 * WAVES) void k_qkv(QkvArgs a) {
  static_assert(R % 2 == 0, "rotary pairs need an even row count per wave");
  extern __shared__ float xs[];  // [0, n): embedding half; [n, 2n): hidden half
  __shared__ float red[32];
  __shared__ float sv[16];
  __shared__ int si[16], st[16];
  const int n = a.n;
  const int N = (a.n_head + 2 * a.n_head_kv) * a.head_dim;
  const int wv = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * WAVES + wv) * R;

  // the first weight loads of the hidden half go out before anything else, so
  // the prologue below (staging, the previous step's argmax, the embedding row)
  // overlaps the weight stream
  uint4 wpf[U][R];
  const bool issued = row0 < N && (n >> 3) >= 64 * U;
  if (issued) rows_issue<R, U>(a.w_qkv, size_t(2) * n, row0, N, n, wpf);
  // hidden half: already weighted by hidden_norm; its sum of squares from partials
  stage_plain(xs + n, a.gw, n);
  float sg = sum_partials(a.g_ssq, a.g_ssq_count);
  const int tok = qkv_token(a, sv, si, st);
  __syncthreads();  // hidden half staged
  // the embedding row and input_layernorm go to registers; they land while the
  // hidden half streams
  const uint2* e4 = reinterpret_cast<const uint2*>(a.embed + (size_t)tok * n);
  const float4* w4 = reinterpret_cast<const float4*>(a.w_in);
  const int n4 = n >> 2;
  uint2 er[kQkvERegs];
  float4 wr[kQkvERegs];
  const bool in_regs = n4 <= kQkvERegs * int(blockDim.x);
#pragma unroll
  for (int j = 0; j < kQkvERegs; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (in_regs && i < n4) {
      er[j] = e4[i];
      wr[j] = w4[i];
    }
  }
  float acc_g[R], acc_e[R];
  if (issued) rows_dot_issued<R, U>(a.w_qkv, size_t(2) * n, row0, N, n, n, xs + n, wpf, acc_g);
  else if (row0 < N) rows_dot<R, U>(a.w_qkv, size_t(2) * n, row0, N, n, n, xs + n, acc_g);
  float se = 0.f;
  float4* x4 = reinterpret_cast<float4*>(xs);
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < kQkvERegs; ++j) {
      const int i = threadIdx.x + j * blockDim.x;
      if (i < n4) {
        const float e0 = bf16_lo(er[j].x), e1 = bf16_hi(er[j].x), e2 = bf16_lo(er[j].y),
                    e3 = bf16_hi(er[j].y);
        x4[i] = make_float4(e0 * wr[j].x, e1 * wr[j].y, e2 * wr[j].z, e3 * wr[j].w);
        se = fmaf(e0, e0, fmaf(e1, e1, fmaf(e2, e2, fmaf(e3, e3, se))));
      }
    }
  } else {
    se = stage_weighted_bf16(xs, a.embed + (size_t)tok * n, a.w_in, n);
  }
  __syncthreads();
  if (row0 < N) rows_dot<R, U>(a.w_qkv, size_t(2) * n, row0, N, 0, n, xs, acc_e);
  block_sum2(se, sg, red);  // every wave takes part
  if (row0 >= N) return;
  const float ie = 1.0f / sqrtf(se / float(n) + a.eps);
  const float ig = 1.0f / sqrtf(sg / float(n) + a.eps);
  qkv_epilogue<R>(a, row0, acc_e, acc_g, ie, ig);
}

constexpr int kQkvGRegs = 5;  // float4 chunks of the hidden half a thread stages at once

// k_qkv with the token table: the table row stands for the embedding half, so only
// the hidden half of W_qkv streams.  Wave loads complete in issue order, so the
// loads the token depends on (the previous step's candidates, one batch of them,
// or the boundary token) go out before the weights: the token is known, and its
// table row and the hidden-half activations requested, while the weights are
// still in flight.  ISSUE: the first U chunk steps of the weights go out before
// the prologue (K / 8 >= 64 U; rows past N repeat the last row).  MORE: more
// candidates than one batch (the later batches load after the weights).
template <int WAVES, int R, int U, bool ISSUE, bool MORE>
__global__ __launch_bounds__(64 * WAVES) void k_qkv_tab(QkvArgs a) {
  static_assert(R % 2 == 0, "rotary pairs need an even row count per wave");
  extern __shared__ float xs[];  // [0, n): hidden half
  __shared__ float red[32];
  __shared__ float sv[16];
  __shared__ int si[16], st[16];
  const int n = a.n;
  const int N = (a.n_head + 2 * a.n_head_kv) * a.head_dim;
  const int wv = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * WAVES + wv) * R;

  // the hidden half's rows: a contiguous copy, or the second halves of W_qkv's rows
  const uint16_t* wh = a.w_hid_rows ? a.w_hid_rows : a.w_qkv + n;
  const size_t ldh = a.w_hid_rows ? size_t(n) : size_t(2) * n;
  ArgmaxBatch first;
  const int tok0 = qkv_token_load(a, first);
  uint4 wpf[U][R];
  if constexpr (ISSUE) rows_issue<R, U>(wh, ldh, row0, N, 0, wpf);
  const int tok = qkv_token_from<MORE>(a, first, tok0, sv, si, st);
  float acc_e[R], acc_g[R];
  const float* trow = a.tok_tab + (size_t)tok * N;  // already divided by rms(E[tok])
#pragma unroll
  for (int r = 0; r < R; ++r) acc_e[r] = trow[min(row0 + r, N - 1)];
  // the hidden half: all of a thread's loads go out together (clamped indices; a
  // clamped store rewrites the last chunk with its own value), so it lands one
  // round trip after the weights at most
  {
    const float4* g4 = reinterpret_cast<const float4*>(a.gw);
    float4* x4 = reinterpret_cast<float4*>(xs);
    const int n4 = n >> 2;
    float4 gr[kQkvGRegs];
#pragma unroll
    for (int j = 0; j < kQkvGRegs; ++j) gr[j] = g4[min(int(threadIdx.x + j * blockDim.x), n4 - 1)];
#pragma unroll
    for (int j = 0; j < kQkvGRegs; ++j) x4[min(int(threadIdx.x + j * blockDim.x), n4 - 1)] = gr[j];
    for (int i = threadIdx.x + kQkvGRegs * blockDim.x; i < n4; i += blockDim.x) x4[i] = g4[i];
  }
  float sg = sum_partials(a.g_ssq, a.g_ssq_count);
  __syncthreads();  // hidden half staged
  if constexpr (ISSUE) rows_dot_issued<R, U>(wh, ldh, row0, N, 0, n, xs, wpf, acc_g);
  else rows_dot<R, U>(wh, ldh, row0, N, 0, n, xs, acc_g);
  float zero = 0.f;
  block_sum2(zero, sg, red);  // every wave takes part
  if (row0 >= N) return;
  const float ig = 1.0f / sqrtf(sg / float(n) + a.eps);
  qkv_epilogue<R>(a, row0, acc_e, acc_g, 1.0f, ig);
}

// k_qkv_q with the token table: only the hidden half's codes stream and only the
// hidden half is quantised; the table row stands for the embedding half.  The
// token's loads go out first (a wave's loads complete in issue order).
template <int WAVES, int R, int U>
__global__ __launch_bounds__(64 * WAVES, kI4WavesPerSimd) void k_qkv_q_tab(QkvArgs a) {
  static_assert(R % 2 == 0, "rotary pairs need an even row count per wave");
  extern __shared__ float xs[];  // [0, n) hidden half, then its quantised planes
  __shared__ float red[32];
  __shared__ float sv[16];
  __shared__ int si[16], st[16];
  const int n = a.n;
  const int N = (a.n_head + 2 * a.n_head_kv) * a.head_dim;
  const int wv = threadIdx.x >> 6;
  const uint8_t* Q = reinterpret_cast<const uint8_t*>(a.w_qkv);
  const size_t ldw = size_t(2) * n;
  const int nvb = (N + WAVES * R - 1) / (WAVES * R);
  ArgmaxBatch first;
  const int tok0 = qkv_token_load(a, first);
  QLoad<R, U> Lg;
  int row0 = (blockIdx.x * WAVES + wv) * R;
  if (row0 < N) q_issue<R, U>(Q, a.s_qkv, ldw, row0, N, n, n, Lg);
  uint4* xpg = reinterpret_cast<uint4*>(xs + n);
  int* xeg = reinterpret_cast<int*>(xpg + n / 8);
  stage_plain(xs, a.gw, n);
  float sg = sum_partials(a.g_ssq, a.g_ssq_count);
  const int tok = qkv_token_from(a, first, tok0, sv, si, st);
  const float* trow = a.tok_tab + (size_t)tok * N;  // already divided by rms(E[tok])
  __syncthreads();  // hidden half staged
  quant_x_i4(xs, n, xpg, xeg);
  float zero = 0.f;
  block_sum2(zero, sg, red);  // its barriers also publish the quantised vector
  const float ig = 1.0f / sqrtf(sg / float(n) + a.eps);
  for (int vb = blockIdx.x;; vb += gridDim.x) {
    if (row0 < N) {
      float acc_g[R], acc_e[R];
      q_dot_issued<R, U>(Q, a.s_qkv, ldw, row0, N, n, n, Lg, xpg, xeg, acc_g);
#pragma unroll
      for (int r = 0; r < R; ++r) acc_e[r] = trow[min(row0 + r, N - 1)];
      qkv_epilogue<R>(a, row0, acc_e, acc_g, 1.0f, ig);
    }
    const int vn = vb + int(gridDim.x);
    if (vn >= nvb) break;
    row0 = (vn * WAVES + wv) * R;
    if (row0 < N) q_issue<R, U>(Q, a.s_qkv, ldw, row0, N, n, n, Lg);
  }
}

// k_qkv with int4 weights: the first row set's codes of both halves go out first;
// both halves are then staged and quantised once per block, and the block covers
// its virtual blocks of rows
template <int WAVES, int R, int U>
__global__ __launch_bounds__(64 * WAVES, kI4WavesPerSimd) void k_qkv_q(QkvArgs a) {
  static_assert(R % 2 == 0, "rotary pairs need an even row count per wave");
  extern __shared__ float xs[];  // [0, n) embedding half, [n, 2n) hidden half, then
                                 // the two quantised halves
  __shared__ float red[32];
  __shared__ float sv[16];
  __shared__ int si[16], st[16];
  const int n = a.n;
  const int N = (a.n_head + 2 * a.n_head_kv) * a.head_dim;
  const int wv = threadIdx.x >> 6;
  const uint8_t* Q = reinterpret_cast<const uint8_t*>(a.w_qkv);
  const size_t ldw = size_t(2) * n;
  const int nvb = (N + WAVES * R - 1) / (WAVES * R);
  QLoad<R, U> Lg, Le;
  int row0 = (blockIdx.x * WAVES + wv) * R;
  if (row0 < N) {
    q_issue<R, U>(Q, a.s_qkv, ldw, row0, N, n, n, Lg);
    q_issue<R, U>(Q, a.s_qkv, ldw, row0, N, 0, n, Le);
  }
  uint4* xpe = reinterpret_cast<uint4*>(xs + 2 * n);
  int* xee = reinterpret_cast<int*>(xpe + n / 8);
  uint4* xpg = reinterpret_cast<uint4*>(xee + n / 32);
  int* xeg = reinterpret_cast<int*>(xpg + n / 8);
  stage_plain(xs + n, a.gw, n);
  float sg = sum_partials(a.g_ssq, a.g_ssq_count);
  const int tok = qkv_token(a, sv, si, st);
  float se = stage_weighted_bf16(xs, a.embed + (size_t)tok * n, a.w_in, n);
  __syncthreads();
  quant_x_i4(xs, n, xpe, xee);
  quant_x_i4(xs + n, n, xpg, xeg);
  block_sum2(se, sg, red);  // its barriers also publish the quantised halves
  const float ie = 1.0f / sqrtf(se / float(n) + a.eps);
  const float ig = 1.0f / sqrtf(sg / float(n) + a.eps);
  for (int vb = blockIdx.x;; vb += gridDim.x) {
    if (row0 < N) {
      float acc_g[R], acc_e[R];
      q_dot_issued<R, U>(Q, a.s_qkv, ldw, row0, N, n, n, Lg, xpg, xeg, acc_g);
      q_dot_issued<R, U>(Q, a.s_qkv, ldw, row0, N, 0, n, Le, xpe, xee, acc_e);
      qkv_epilogue<R>(a, row0, acc_e, acc_g, ie, ig);
    }
    const int vn = vb + int(gridDim.x);
    if (vn >= nvb) break;
    row0 = (vn * WAVES + wv) * R;
    if (row0 < N) {
      q_issue<R, U>(Q, a.s_qkv, ldw, row0, N, n, n, Lg);
      q_issue<R, U>(Q, a.s_qkv, ldw, row0, N, 0, n, Le);
    }
  }
}

// ---------------------------------------------------------------------------
template <int WAVES, int R, int U, bool I4>
__global__ __launch_bounds__(64 * WAVES, I4 ? kI4WavesPerSimd : 1) void k_gemv_resid(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ S, int N, int K,
    const float* __restrict__ x, const float* __restrict__ resid, VecOut out) {
  extern __shared__ float xs[];  // [K]; int4: then the quantised vector
  __shared__ float red[16];
  const int wv = threadIdx.x >> 6;
  auto finish = [&](float (&acc)[R], int row0) {
    if (row0 < N) {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += resid[min(row0 + r, N - 1)];
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
    }
  };
  if constexpr (!I4) {
    stage_plain(xs, x, K);
    __syncthreads();
    const int row0 = (blockIdx.x * WAVES + wv) * R;
    float acc[R];
    if (row0 < N) rows_dot<R, U>(W, size_t(K), row0, N, 0, K, xs, acc);
    finish(acc, row0);
    emit_rows<R, WAVES>(acc, row0, N, out, red, blockIdx.x);
  } else {
    const uint8_t* Q = reinterpret_cast<const uint8_t*>(W);
    const int nvb = (N + WAVES * R - 1) / (WAVES * R);
    QLoad<R, U> L;
    int row0 = (blockIdx.x * WAVES + wv) * R;
    if (row0 < N) q_issue<R, U>(Q, S, size_t(K), row0, N, 0, K, L);
    stage_plain(xs, x, K);
    __syncthreads();
    uint4* xp = reinterpret_cast<uint4*>(xs + K);
    int* xe = reinterpret_cast<int*>(xp + K / 8);
    quant_x_i4(xs, K, xp, xe);
    __syncthreads();
    for (int vb = blockIdx.x;; vb += gridDim.x) {
      float acc[R];
      if (row0 < N) q_dot_issued<R, U>(Q, S, size_t(K), row0, N, 0, K, L, xp, xe, acc);
      finish(acc, row0);
      emit_rows<R, WAVES>(acc, row0, N, out, red, vb);
      const int vn = vb + int(gridDim.x);
      if (vn >= nvb) break;
      __syncthreads();  // red is reused by the next virtual block
      row0 = (vn * WAVES + wv) * R;
      if (row0 < N) q_issue<R, U>(Q, S, size_t(K), row0, N, 0, K, L);
    }
  }
}

// ---------------------------------------------------------------------------
template <int WAVES, int R, int U, bool I4>
__global__ __launch_bounds__(64 * WAVES, I4 ? kI4WavesPerSimd : 1) void k_gateup(const uint16_t* __restrict__ W,
                                                       const uint16_t* __restrict__ S, int n_ff,
                                                       int n, const float* __restrict__ xw,
                                                       const float* __restrict__ x_ssq,
                                                       int ssq_count, float eps,
                                                       float* __restrict__ act) {
  static_assert(R % 2 == 0, "gate/up pairs need an even row count per wave");
  extern __shared__ float xs[];  // [n]; int4: then the quantised vector
  __shared__ float red[32];
  const int N = 2 * n_ff;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  QLoad<(I4 ? R : 1), (I4 ? U : 1)> L0;  // int4: the first row set, loaded before the stage
  if constexpr (I4) {
    const int row0 = (blockIdx.x * WAVES + wv) * R;
    if (row0 < N) q_issue<R, U>(reinterpret_cast<const uint8_t*>(W), S, size_t(n), row0, N, 0, n, L0);
  }
  stage_plain(xs, xw, n);
  float ss = sum_partials(x_ssq, ssq_count), dummy = 0.f;
  __syncthreads();
  auto epilogue = [&](int row0, const float (&acc)[R], float inv) {
#pragma unroll
    for (int p = 0; p < R / 2; ++p) {
      const int r = row0 + 2 * p;
      if (lane == p && r < N) {
        const float gt = acc[2 * p] * inv, up = acc[2 * p + 1] * inv;
        act[r >> 1] = (gt / (1.0f + expf(-gt))) * up;
      }
    }
  };
  if constexpr (!I4) {
    const int row0 = (blockIdx.x * WAVES + wv) * R;
    float acc[R];
    if (row0 < N) rows_dot<R, U>(W, size_t(n), row0, N, 0, n, xs, acc);
    block_sum2(ss, dummy, red);
    if (row0 >= N) return;
    epilogue(row0, acc, 1.0f / sqrtf(ss / float(n) + eps));
  } else {
    uint4* xp = reinterpret_cast<uint4*>(xs + n);
    int* xe = reinterpret_cast<int*>(xp + n / 8);
    quant_x_i4(xs, n, xp, xe);
    block_sum2(ss, dummy, red);  // its barriers also publish the quantised vector
    const float inv = 1.0f / sqrtf(ss / float(n) + eps);
    const uint8_t* Q = reinterpret_cast<const uint8_t*>(W);
    const int nvb = (N + WAVES * R - 1) / (WAVES * R);
    int row0 = (blockIdx.x * WAVES + wv) * R;
    for (int vb = blockIdx.x;; vb += gridDim.x) {
      const int vn = vb + int(gridDim.x), rn = (vn * WAVES + wv) * R;
      QLoad<R, U> Ln;
      if (vn < nvb && rn < N) q_issue<R, U>(Q, S, size_t(n), rn, N, 0, n, Ln);
      if (row0 < N) {
        float acc[R];
        q_dot_issued<R, U>(Q, S, size_t(n), row0, N, 0, n, L0, xp, xe, acc);
        epilogue(row0, acc, inv);
      }
      if (vn >= nvb) break;
      L0 = Ln;
      row0 = rn;
    }
  }
}

// ---------------------------------------------------------------------------
// The block's lm_head candidate for virtual block vb from its waves' R logits each:
// the best (value, index) (lowest index on ties) and, with d2t, that index's target
// id; dt is lane r's d2t of row row0 + r.  Every thread of the block calls it.
template <int R, int WAVES>
__device__ __forceinline__ void lm_candidates(const LmHeadArgs& a, const float (&acc)[R], int row0, float inv,
                                              int dt, int vb, float* bv_s, int* bi_s, int* bt_s) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF, br = 0;
  if (row0 < a.dv) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (row0 + r < a.dv) {
        const float v = acc[r] * inv;
        if (better(v, row0 + r, bv, bi)) { bv = v; bi = row0 + r; br = r; }
        if (a.logits_dbg && lane == r) a.logits_dbg[row0 + r] = v;
      }
    }
  }
  int bt = bi + __shfl(dt, br, kWave);
  if (lane == 0) { bv_s[wv] = bv; bi_s[wv] = bi; bt_s[wv] = bt; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < WAVES; ++w)
      if (better(bv_s[w], bi_s[w], bv, bi)) { bv = bv_s[w]; bi = bi_s[w]; bt = bt_s[w]; }
    a.part_val[vb] = bv;
    a.part_idx[vb] = bi;
    if (a.d2t) a.part_tok[vb] = bt;
  }
}

// d2t of a wave's rows (lane r holds row0 + r's)
template <int R>
__device__ __forceinline__ int lm_d2t_of(const LmHeadArgs& a, int row0) {
  const int lane = threadIdx.x & 63;
  return (a.d2t && lane < R && row0 + lane < a.dv) ? a.d2t[row0 + lane] : 0;
}

// one block of the bf16 lm_head: rows [bid * WAVES * R, ...), candidate slot bid
template <int WAVES, int R, int U>
__device__ __forceinline__ void lmhead_bf16(const LmHeadArgs& a, int bid, float* xs, float* red, float* bv_s,
                                            int* bi_s, int* bt_s) {
  const int wv = threadIdx.x >> 6;
  const int row0 = (bid * WAVES + wv) * R;
  const int dt = lm_d2t_of<R>(a, row0);  // loaded before the stream
  stage_plain(xs, a.hw, a.n);
  float ss = sum_partials(a.h_ssq, a.h_ssq_count), dummy = 0.f;
  __syncthreads();
  float acc[R];
  if (row0 < a.dv) rows_dot<R, U>(a.w_lm, size_t(a.n), row0, a.dv, 0, a.n, xs, acc);
  block_sum2(ss, dummy, red);
  lm_candidates<R, WAVES>(a, acc, row0, 1.0f / sqrtf(ss / float(a.n) + a.eps), dt, bid, bv_s, bi_s, bt_s);
}

// The int4 lm_head's blocks: block bid of nblk covers virtual blocks (candidate slots)
// bid, bid + nblk, ... of the dv rows
template <int WAVES, int R, int U>
__device__ __forceinline__ void lmhead_i4(const LmHeadArgs& a, int bid, int nblk, float* xs, float* red,
                                          float* bv_s, int* bi_s, int* bt_s) {
  {
    const int wv = threadIdx.x >> 6;
    int row0 = (bid * WAVES + wv) * R;
    const uint8_t* Q = reinterpret_cast<const uint8_t*>(a.w_lm);
    const size_t ldw = size_t(a.n);
    const int nvb = (a.dv + WAVES * R - 1) / (WAVES * R);
    QLoad<R, U> L;
    if (row0 < a.dv) q_issue<R, U>(Q, a.s_lm, ldw, row0, a.dv, 0, a.n, L);
    int dt = lm_d2t_of<R>(a, row0);
    stage_plain(xs, a.hw, a.n);
    float ss = sum_partials(a.h_ssq, a.h_ssq_count), dummy = 0.f;
    __syncthreads();
    uint4* xp = reinterpret_cast<uint4*>(xs + a.n);
    int* xe = reinterpret_cast<int*>(xp + a.n / 8);
    quant_x_i4(xs, a.n, xp, xe);
    block_sum2(ss, dummy, red);  // its barriers also publish the quantised vector
    const float inv = 1.0f / sqrtf(ss / float(a.n) + a.eps);
    for (int vb = bid;; vb += nblk) {
      const int vn = vb + nblk, rn = (vn * WAVES + wv) * R;
      QLoad<R, U> Ln;
      int dtn = 0;
      if (vn < nvb) {
        if (rn < a.dv) q_issue<R, U>(Q, a.s_lm, ldw, rn, a.dv, 0, a.n, Ln);
        dtn = lm_d2t_of<R>(a, rn);
      }
      float acc[R];
      if (row0 < a.dv) q_dot_issued<R, U>(Q, a.s_lm, ldw, row0, a.dv, 0, a.n, L, xp, xe, acc);
      lm_candidates<R, WAVES>(a, acc, row0, inv, dt, vb, bv_s, bi_s, bt_s);
      if (vn >= nvb) break;
      __syncthreads();  // the candidate slots are reused
      L = Ln;
      row0 = rn;
      dt = dtn;
    }
  }
}

template <int WAVES, int R, int U, bool I4>
__global__ __launch_bounds__(64 * WAVES, I4 ? kI4WavesPerSimd : 1) void k_lmhead(LmHeadArgs a) {
  extern __shared__ float xs[];  // [n]; int4: then the quantised vector
  __shared__ float red[32];
  __shared__ float bv_s[16];
  __shared__ int bi_s[16], bt_s[16];
  if constexpr (!I4) {
    lmhead_bf16<WAVES, R, U>(a, blockIdx.x, xs, red, bv_s, bi_s, bt_s);
  } else {
    lmhead_i4<WAVES, R, U>(a, blockIdx.x, gridDim.x, xs, red, bv_s, bi_s, bt_s);
  }
}

// The next step's hidden-half QKV sums (QhArgs, scaled by 1/rms(g)) in the first qb
// blocks, the bf16 lm_head in the rest: two independent weight streams in one launch.
// ISSUE (the hidden half alone, one wave of blocks): the first U chunk steps of the
// weights go out before g is staged (K / 8 >= 64 U).
// One block's hidden-half QKV sums: each wave owns R rows of the N hidden-half rows
// (ISSUE: its first U chunk steps are in flight before gw is staged)
template <int WAVES, int R, int U, bool ISSUE>
__device__ __forceinline__ void qh_block(const QhArgs& q, int bid, float* xs, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row0 = (bid * WAVES + wv) * R;
  uint4 wpf[ISSUE ? U : 1][R];
  if constexpr (ISSUE) rows_issue<R, U>(q.w, q.ldw, row0, q.N, 0, wpf);
  stage_plain(xs, q.gw, q.n);
  float sg = sum_partials(q.g_ssq, q.g_ssq_count), dummy = 0.f;
  __syncthreads();
  float acc[R];
  if constexpr (ISSUE) rows_dot_issued<R, U>(q.w, q.ldw, row0, q.N, 0, q.n, xs, wpf, acc);
  else if (row0 < q.N) rows_dot<R, U>(q.w, q.ldw, row0, q.N, 0, q.n, xs, acc);
  block_sum2(sg, dummy, red);  // every wave takes part
  if (row0 >= q.N) return;
  const float ig = 1.0f / sqrtf(sg / float(q.n) + q.eps);
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (lane == r && row0 + r < q.N) q.hsum[row0 + r] = acc[r] * ig;
}

template <int WAVES, int R, int U, bool ISSUE>
__global__ __launch_bounds__(64 * WAVES) void k_lmhead_qh(LmHeadArgs a, QhArgs q, int qb) {
  extern __shared__ float xs[];  // [n]
  __shared__ float red[32];
  __shared__ float bv_s[16];
  __shared__ int bi_s[16], bt_s[16];
  if (int(blockIdx.x) >= qb) {
    lmhead_bf16<WAVES, R, U>(a, int(blockIdx.x) - qb, xs, red, bv_s, bi_s, bt_s);
    return;
  }
  qh_block<WAVES, R, U, ISSUE>(q, int(blockIdx.x), xs, red);
}

// The int4 hidden-half sums of virtual blocks bid, bid + qb, ... (of nvq; WAVES x R
// rows each): g staged and quantised once per block, each virtual block's first U
// chunk steps issued before the previous one's products
template <int WAVES, int R, int U>
__device__ __forceinline__ void qh_i4_block(const QhArgs& q, int bid, int qb, int nvq, float* xs, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint8_t* Q = reinterpret_cast<const uint8_t*>(q.w);
  int row0 = (bid * WAVES + wv) * R;
  QLoad<R, U> L;
  if (row0 < q.N) q_issue<R, U>(Q, q.s, q.ldw, row0, q.N, q.k0, q.n, L);
  stage_plain(xs, q.gw, q.n);
  float sg = sum_partials(q.g_ssq, q.g_ssq_count), dummy = 0.f;
  __syncthreads();
  uint4* xp = reinterpret_cast<uint4*>(xs + q.n);
  int* xe = reinterpret_cast<int*>(xp + q.n / 8);
  quant_x_i4(xs, q.n, xp, xe);
  block_sum2(sg, dummy, red);  // its barriers also publish the quantised vector
  const float ig = 1.0f / sqrtf(sg / float(q.n) + q.eps);
  for (int vb = bid;; vb += qb) {
    const int vn = vb + qb, rn = (vn * WAVES + wv) * R;
    QLoad<R, U> Ln;
    if (vn < nvq && rn < q.N) q_issue<R, U>(Q, q.s, q.ldw, rn, q.N, q.k0, q.n, Ln);
    if (row0 < q.N) {
      float acc[R];
      q_dot_issued<R, U>(Q, q.s, q.ldw, row0, q.N, q.k0, q.n, L, xp, xe, acc);
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == r && row0 + r < q.N) q.hsum[row0 + r] = acc[r] * ig;
    }
    if (vn >= nvq) break;
    L = Ln;
    row0 = rn;
  }
}

// k_lmhead_qh with int4 weights: the first qb blocks cover the nvq virtual blocks of
// hidden-half rows (int4 codes of columns k0 .. k0 + n; g quantised once per block),
// the next lb blocks the int4 lm_head's nvl virtual blocks (candidate slots)
template <int WAVES, int R, int U>
__global__ __launch_bounds__(64 * WAVES, kI4WavesPerSimd) void k_lmhead_qh_i4(LmHeadArgs a, QhArgs q, int qb,
                                                                                int nvq, int lb) {
  extern __shared__ float xs[];  // [n], then the quantised vector
  __shared__ float red[32];
  __shared__ float bv_s[16];
  __shared__ int bi_s[16], bt_s[16];
  if (int(blockIdx.x) >= qb) {
    lmhead_i4<WAVES, R, U>(a, int(blockIdx.x) - qb, lb, xs, red, bv_s, bi_s, bt_s);
    return;
  }
  qh_i4_block<WAVES, R, U>(q, int(blockIdx.x), qb, nvq, xs, red);
}

// the last step of a chain: argmax over the lm_head candidates, d2t (the
// candidates' target ids come with them when pt is given)
__global__ __launch_bounds__(256) void k_argmax_finalize(uint32_t* __restrict__ status,
                                                         const float* __restrict__ pv,
                                                         const int32_t* __restrict__ pi,
                                                         const int32_t* __restrict__ pt, int count,
                                                         const int32_t* __restrict__ d2t, int dv,
                                                         int32_t* out_id, int32_t* tok_store) {
  __shared__ float sv[16];
  __shared__ int si[16], st[16];
  int bt;
  const int bi = block_argmax_carry(pv, pi, pt, count, sv, si, st, &bt);
  if (threadIdx.x == 0) {
    int t;
    if (bi < 0 || bi >= dv) {  // every logit NaN
      t = d2t[0];
      atomicOr(status, kStatusNanLogits);
    } else {
      t = pt ? bt : bi + d2t[bi];
    }
    *out_id = t;
    if (tok_store) *tok_store = t;
  }
}

// ---------------------------------------------------------------------------
// Multi-vector split-K GEMV: P[z][m][r] = sum_{k in chunk z} W[r, k] * X_m[k]
// for m < M.  X is either three fp32 tap streams concatenated along K (x0/x1/x2
// with row length seg) or one fp32 matrix (x1 == nullptr) with row stride K.
// Each weight chunk is loaded once and applied to all M vectors; a block covers
// 8 * R rows, with R chosen so the accumulators stay in registers.
template <int M>
struct MultiShape {
  static constexpr int R = M <= 4 ? 8 : (M <= 8 ? 4 : 2);
  static constexpr int WAVES = 8;
  static constexpr int ROWS = WAVES * R;
};

// one block: row block bx of the weights over K chunk z; xs holds [M][kc] floats
template <int M, bool I4>
__device__ __forceinline__ void gemv_multi_block(int bx, int z, const uint16_t* __restrict__ W,
                                                 const uint16_t* __restrict__ S, int N, int K, int kc,
                                                 const float* __restrict__ x0, const float* __restrict__ x1,
                                                 const float* __restrict__ x2, int seg, int rows,
                                                 float* __restrict__ P, const TapRowsB& yb, float* xs) {
  constexpr int R = MultiShape<M>::R;
  constexpr int WAVES = MultiShape<M>::WAVES;
  constexpr int NT = 64 * WAVES;
  const int k0 = z * kc;
  const int klen = min(kc, K - k0);
  const int k4 = klen >> 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row0 = (bx * WAVES + wv) * R;
  const int nch = I4 ? (klen >> 5) : (klen >> 3);  // 16-byte chunks of the K range
  const uint4* wp[R];
  const uint16_t* sp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t row = (size_t)min(row0 + r, N - 1);
    if constexpr (I4) {
      wp[r] = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(W) + row * (K / 2) + k0 / 2);
      sp[r] = S + row * (K / 32) + k0 / 32;
    } else {
      wp[r] = reinterpret_cast<const uint4*>(W + row * K + k0);
      sp[r] = nullptr;
    }
  }
  // element k of vector m (fp32): from the tap streams or one matrix
  auto src_of = [&](int m, int k) -> const float* {
    if (x1) {
      const int sgi = k / seg;
      // rows from yb.rows_x on come from the second set of streams
      const bool second = m >= yb.rows_x;
      const float* base = second ? (sgi == 0 ? yb.y[0] : (sgi == 1 ? yb.y[1] : yb.y[2]))
                                 : (sgi == 0 ? x0 : (sgi == 1 ? x1 : x2));
      return base + (size_t)(second ? m - yb.rows_x : m) * seg + (k - sgi * seg);
    }
    return x0 + (size_t)m * K + k;
  };
  // int4: each vector's chunk in five-digit fixed point per group of 32, quantised
  // straight from the sources once per block (planes [M][4][G] uint4, plane 4
  // [M][G] uint4, exponents [M][G]); bf16: the M vectors staged as floats
  uint4* xpl = reinterpret_cast<uint4*>(xs);
  uint4* xp4 = xpl + (size_t)M * (kc >> 3);
  int* xex = reinterpret_cast<int*>(xp4 + (size_t)M * (kc >> 5));
  if constexpr (I4) {
    const int nq = klen >> 3, G = klen >> 5, total = M * nq;  // nq % 4 == 0: quads stay in one vector
    for (int j0 = 0; j0 < total; j0 += NT) {  // same trip count for every lane
      const int j = j0 + int(threadIdx.x);
      const int m = j / nq, jj = j - m * nq;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (j < total && m < rows) {
        const float* p = src_of(m, k0 + 8 * jj);
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
      }
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint4 pl;
      uint32_t p4;
      int e;
      quant8_5(v, pl, p4, e);
      if (j < total) {
        xpl[(size_t)m * (kc >> 3) + (jj & 3) * G + (jj >> 2)] = pl;
        reinterpret_cast<uint32_t*>(xp4 + (size_t)m * (kc >> 5))[jj] = p4;
        if ((jj & 3) == 0) xex[m * (kc >> 5) + (jj >> 2)] = e;
      }
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(xs);
    const int total = M * k4;
#pragma unroll 4
    for (int idx = threadIdx.x; idx < total; idx += NT) {
      const int m = idx / k4, i = idx - m * k4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < rows) v = *reinterpret_cast<const float4*>(src_of(m, k0 + 4 * i));
      dst[(size_t)m * (kc >> 2) + i] = v;
    }
  }
  __syncthreads();
  if (row0 >= N) return;
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
  auto apply = [&](int c, const uint4 (&w)[R]) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* x4 = reinterpret_cast<const float4*>(xs + m * kc);
      const float4 a = x4[2 * c], b = x4[2 * c + 1];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][m] = dot8(w[r], a, b, acc[r][m]);
    }
  };
  if constexpr (I4) {
    // group c: v_dot8 of each row's 32 codes with each vector's five digit planes,
    // scaled by the row's scale and the vector's 2^-e (q_group5)
    const int G = nch;
    for (int c = lane; c < nch; c += 64) {
      uint4 w[R];
      uint16_t sc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[r] = ld_stream(wp[r] + c);
        sc[r] = sp[r][c];
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float am[R];
#pragma unroll
        for (int r = 0; r < R; ++r) am[r] = acc[r][m];
        q_group5<R>(w, sc, c, G, xpl + (size_t)m * (kc >> 3), xp4 + (size_t)m * (kc >> 5), xex + m * (kc >> 5),
                    am);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][m] = am[r];
      }
    }
  } else {
    for (int c = lane; c < nch; c += 64) {
      uint4 w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = ld_stream(wp[r] + c);
      apply(c, w);
    }
  }
  // the R * M sums: one reduce-scatter over the wave (padded with zeros to a power
  // of two), then one store per lane group
  constexpr int NVAL = R * M;
  static_assert(NVAL <= 32, "accumulators per lane");
  constexpr int NV = NVAL <= 8 ? 8 : (NVAL <= 16 ? 16 : 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = i < NVAL ? acc[(i % NVAL) / M][(i % NVAL) % M] : 0.f;
  wave_reduce_scatter<NV>(v);
  constexpr int GL = 64 / NV;
  const int j = lane / GL;
  if (lane % GL == 0 && j < NVAL) {
    const int r = j / M, m = j - r * M;
    if (row0 + r < N) P[((size_t)z * M + m) * N + row0 + r] = v[0];
  }
}

template <int M, bool I4>
__global__ __launch_bounds__(512) void k_gemv_multi(const uint16_t* __restrict__ W,
                                                    const uint16_t* __restrict__ S, int N, int K,
                                                    int kc, const float* __restrict__ x0,
                                                    const float* __restrict__ x1,
                                                    const float* __restrict__ x2, int seg,
                                                    int rows, float* __restrict__ P,
                                                    const TapRowsB yb) {
  static_assert(MultiShape<M>::WAVES == 8, "512 threads");
  extern __shared__ float xs[];  // [M][kc]
  gemv_multi_block<M, I4>(int(blockIdx.x), int(blockIdx.y), W, S, N, K, kc, x0, x1, x2, seg, rows, P, yb, xs);
}

// The K/V rows of a teacher-forced pass (bf16 weights, one fp32 activation matrix)
// and, in the same launch, the hidden-half QKV sums of the boundary feature the pass
// writes (the next chain's first step; qh_block in its 8-wave, 2-row form): blocks
// [0, qb) the sums, the rest the (row block, K chunk) grid of the multi-vector GEMV,
// gx row blocks per chunk
template <int M>
__global__ __launch_bounds__(512) void k_gemv_multi_qh(const uint16_t* __restrict__ W, int N, int K, int kc,
                                                       const float* __restrict__ x0, int rows,
                                                       float* __restrict__ P, QhArgs q, int qb, int gx) {
  static_assert(MultiShape<M>::WAVES == 8, "512 threads");
  extern __shared__ float xs[];  // [max(M * kc, n)]
  __shared__ float red[32];
  const int b = int(blockIdx.x);
  if (b < qb) {
    qh_block<8, 2, 4, false>(q, b, xs, red);
    return;
  }
  const int t = b - qb;
  const TapRowsB none{{nullptr, nullptr, nullptr}, 1 << 30};
  gemv_multi_block<M, false>(t % gx, t / gx, W, nullptr, N, K, kc, x0, nullptr, nullptr, 0, rows, P, none, xs);
}

// ---------------------------------------------------------------------------
// launchers: the configuration (waves per block, rows per wave, chunk steps in
// flight) is picked per matrix shape from the tuned table in gemv_cfg.hpp
#define E3_DISPATCH_CFG(cfg, CASE)                                                \
  switch (cfg) {                                                                  \
    E3_GEMV_CONFIGS(CASE)                                                         \
    default:                                                                      \
      return hipErrorInvalidValue;                                                \
  }

static inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// raise a kernel's dynamic LDS limit to `bytes` (once per kernel and size; the int4
// kernels stage the vector and its quantised form, which can pass 64 KB)
template <auto F>
static hipError_t lds_allow(size_t bytes) {
  static size_t allowed = 64 * 1024;
  if (bytes <= allowed) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(F),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e == hipSuccess) allowed = bytes;
  return e;
}
#define E3_LDS_ALLOW(KERNEL, BYTES)                                \
  do {                                                             \
    const hipError_t _e = lds_allow<KERNEL>(BYTES);                \
    if (_e != hipSuccess) return _e;                               \
  } while (0)

int gemv_grid(int N, int cfg) {
  switch (cfg) {
#define CASE(ID, WV, RR, UU) \
  case ID:                   \
    return ceil_div(N, WV * RR);
    E3_GEMV_CONFIGS(CASE)
#undef CASE
    default:
      return -1;
  }
}

// (S non-null: W holds int4 codes and S their scales)
hipError_t launch_encode(const uint16_t* w_fc, const uint16_t* S, int n, const float* a0,
                         const float* a1, const float* a2, const VecOut& out, int cfg,
                         hipStream_t s) {
  const size_t xb = size_t(3 * n) * sizeof(float);
#define CASE(ID, WV, RR, UU)                                                                    \
  case ID:                                                                                      \
    if (S) {                                                                                    \
      E3_LDS_ALLOW((k_encode<WV, RR, UU, true>), xb + q_vec_bytes(3 * n));                      \
      E3_LAUNCH((k_encode<WV, RR, UU, true>), dim3(i4_grid(ceil_div(n, WV * RR))),     \
                         dim3(64 * WV), xb + q_vec_bytes(3 * n), s, w_fc, S, n, a0, a1, a2, out); \
    } else                                                                                      \
      E3_LAUNCH((k_encode<WV, RR, UU, false>), dim3(ceil_div(n, WV * RR)), dim3(64 * WV), \
                         xb, s, w_fc, S, n, a0, a1, a2, out);                                   \
    break;
  E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
  return hipGetLastError();
}

hipError_t launch_qkv(const QkvArgs& a, int cfg, hipStream_t s) {
  const int N = (a.n_head + 2 * a.n_head_kv) * a.head_dim;
  const size_t xb = size_t(2 * a.n) * sizeof(float);
#define CASE(ID, WV, RR, UU)                                                               \
  case ID:                                                                                 \
    if (RR % 2) return hipErrorInvalidValue;                                               \
    if (a.s_qkv && a.tok_tab) {                                                            \
      E3_LDS_ALLOW((k_qkv_q_tab<WV, (RR < 2 ? 2 : RR), UU>), xb / 2 + q_vec_bytes(a.n));    \
      E3_LAUNCH((k_qkv_q_tab<WV, (RR < 2 ? 2 : RR), UU>), dim3(i4_grid(ceil_div(N, WV * RR))), \
                         dim3(64 * WV), xb / 2 + q_vec_bytes(a.n), s, a);                  \
    } else if (a.s_qkv) {                                                                  \
      E3_LDS_ALLOW((k_qkv_q<WV, (RR < 2 ? 2 : RR), UU>), xb + 2 * q_vec_bytes(a.n));        \
      E3_LAUNCH((k_qkv_q<WV, (RR < 2 ? 2 : RR), UU>), dim3(i4_grid(ceil_div(N, WV * RR))), \
                         dim3(64 * WV), xb + 2 * q_vec_bytes(a.n), s, a);                  \
    } else if (a.tok_tab) {                                                                \
      const bool iss = (a.n >> 3) >= 64 * UU, more = a.prev_count > kArgmaxBatch * 64 * WV;  \
      if (iss && !more)                                                                    \
        E3_LAUNCH((k_qkv_tab<WV, (RR < 2 ? 2 : RR), UU, true, false>), dim3(ceil_div(N, WV * RR)), \
                  dim3(64 * WV), xb / 2, s, a);                                            \
      else if (iss)                                                                        \
        E3_LAUNCH((k_qkv_tab<WV, (RR < 2 ? 2 : RR), UU, true, true>), dim3(ceil_div(N, WV * RR)), \
                  dim3(64 * WV), xb / 2, s, a);                                            \
      else                                                                                 \
        E3_LAUNCH((k_qkv_tab<WV, (RR < 2 ? 2 : RR), UU, false, true>), dim3(ceil_div(N, WV * RR)), \
                  dim3(64 * WV), xb / 2, s, a);                                            \
    }                                                                                      \
    else                                                                                   \
      E3_LAUNCH((k_qkv<WV, (RR < 2 ? 2 : RR), UU>), dim3(ceil_div(N, WV * RR)),   \
                         dim3(64 * WV), xb, s, a);                                         \
    break;
  E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
  return hipGetLastError();
}

hipError_t launch_gemv_resid(const uint16_t* w, const uint16_t* S, int N, int K, const float* x,
                             const float* resid, const VecOut& out, int cfg, hipStream_t s) {
  const size_t xb = size_t(K) * sizeof(float);
#define CASE(ID, WV, RR, UU)                                                                    \
  case ID:                                                                                      \
    if (S) {                                                                                    \
      E3_LDS_ALLOW((k_gemv_resid<WV, RR, UU, true>), xb + q_vec_bytes(K));                      \
      E3_LAUNCH((k_gemv_resid<WV, RR, UU, true>), dim3(i4_grid(ceil_div(N, WV * RR))), \
                         dim3(64 * WV), xb + q_vec_bytes(K), s, w, S, N, K, x, resid, out);    \
    } else                                                                                      \
      E3_LAUNCH((k_gemv_resid<WV, RR, UU, false>), dim3(ceil_div(N, WV * RR)),        \
                         dim3(64 * WV), xb, s, w, S, N, K, x, resid, out);                     \
    break;
  E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
  return hipGetLastError();
}

hipError_t launch_gateup(const uint16_t* w_gu, const uint16_t* S, int n_ff, int n, const float* xw,
                         const float* x_ssq, int ssq_count, float eps, float* act, int cfg,
                         hipStream_t s) {
  const size_t xb = size_t(n) * sizeof(float);
#define CASE(ID, WV, RR, UU)                                                                \
  case ID:                                                                                  \
    if (RR % 2) return hipErrorInvalidValue;                                                \
    if (S) {                                                                                \
      E3_LDS_ALLOW((k_gateup<WV, (RR < 2 ? 2 : RR), UU, true>), xb + q_vec_bytes(n));       \
      E3_LAUNCH((k_gateup<WV, (RR < 2 ? 2 : RR), UU, true>),                       \
                         dim3(i4_grid(ceil_div(2 * n_ff, WV * RR))), dim3(64 * WV),          \
                         xb + q_vec_bytes(n), s, w_gu, S, n_ff, n, xw, x_ssq, ssq_count, eps, act); \
    } else                                                                                  \
      E3_LAUNCH((k_gateup<WV, (RR < 2 ? 2 : RR), UU, false>),                      \
                         dim3(ceil_div(2 * n_ff, WV * RR)), dim3(64 * WV), xb,              \
                         s, w_gu, S, n_ff, n, xw, x_ssq, ssq_count, eps, act);              \
    break;
  E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
  return hipGetLastError();
}

// number of candidate partials (virtual blocks, also with int4 weights)
int lmhead_grid(int dv, int cfg) { return gemv_grid(dv, cfg); }

hipError_t launch_lmhead(const LmHeadArgs& a, int cfg, hipStream_t s) {
  const size_t xb = size_t(a.n) * sizeof(float);
#define CASE(ID, WV, RR, UU)                                                                  \
  case ID:                                                                                    \
    if (a.s_lm) {                                                                             \
      E3_LDS_ALLOW((k_lmhead<WV, RR, UU, true>), xb + q_vec_bytes(a.n));                      \
      E3_LAUNCH((k_lmhead<WV, RR, UU, true>), dim3(i4_grid(ceil_div(a.dv, WV * RR))), \
                         dim3(64 * WV), xb + q_vec_bytes(a.n), s, a);                         \
    } else                                                                                    \
      E3_LAUNCH((k_lmhead<WV, RR, UU, false>), dim3(ceil_div(a.dv, WV * RR)),         \
                         dim3(64 * WV), xb, s, a);                                            \
    break;
  E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
  return hipGetLastError();
}

hipError_t launch_lmhead_qh(const LmHeadArgs& a, const QhArgs& q, int cfg, hipStream_t s) {
  const bool i4 = q.s != nullptr;
  if ((a.w_lm && (a.n != q.n || (a.s_lm != nullptr) != i4)) || (q.n % (i4 ? 32 : 8)) || (q.k0 % (i4 ? 32 : 8)))
    return hipErrorInvalidValue;
  const size_t xb = size_t(q.n) * sizeof(float);
  if (i4) {
#define CASE(ID, WV, RR, UU)                                                                              \
  case ID: {                                                                                              \
    const int nvq = ceil_div(q.N, WV * RR), qb = i4_grid(nvq);                                             \
    const int lb = a.w_lm ? i4_grid(ceil_div(a.dv, WV * RR)) : 0;                                          \
    E3_LDS_ALLOW((k_lmhead_qh_i4<WV, RR, UU>), xb + q_vec_bytes(q.n));                                     \
    E3_LAUNCH((k_lmhead_qh_i4<WV, RR, UU>), dim3(qb + lb), dim3(64 * WV), xb + q_vec_bytes(q.n), s, a, q, qb, \
              nvq, lb);                                                                                   \
  } break;
    E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
    return hipGetLastError();
  }
#define CASE(ID, WV, RR, UU)                                                                 \
  case ID: {                                                                                 \
    const int qb = ceil_div(q.N, WV * RR), lb = a.w_lm ? ceil_div(a.dv, WV * RR) : 0;          \
    if (!a.w_lm && (q.n >> 3) >= 64 * UU)                                                     \
      E3_LAUNCH((k_lmhead_qh<WV, RR, UU, true>), dim3(qb), dim3(64 * WV), xb, s, a, q, qb);     \
    else                                                                                       \
      E3_LAUNCH((k_lmhead_qh<WV, RR, UU, false>), dim3(qb + lb), dim3(64 * WV), xb, s, a, q, qb); \
  } break;
  E3_DISPATCH_CFG(cfg, CASE)
#undef CASE
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(uint32_t* status, const float* pv, const int32_t* pi, const int32_t* pt,
                                  int count, const int32_t* d2t, int dv, int32_t* out_id, int32_t* tok_store,
                                  hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_finalize, dim3(1), dim3(256), 0, s, status, pv, pi, pt, count, d2t, dv, out_id,
                     tok_store);
  return hipGetLastError();
}

// multi-vector: M is rounded up to an instantiated width
int gemv_multi_width(int rows) {
  static const int widths[] = {1, 2, 3, 4, 5, 6, 8, 9, 12, 16};
  for (int w : widths)
    if (rows <= w) return w;
  return -1;
}

static int multi_rows_per_block(int m) {
  switch (m) {
#define RCASE(MM) \
  case MM:        \
    return MultiShape<MM>::ROWS;
    RCASE(1) RCASE(2) RCASE(3) RCASE(4) RCASE(5) RCASE(6) RCASE(8) RCASE(9) RCASE(12) RCASE(16)
#undef RCASE
    default:
      return -1;
  }
}

// K chunk: at most 64 KB of LDS for the M vectors, at least ~512 blocks in all
static int multi_kchunk(int m, int N, int K) {
  const int row_blocks = ceil_div(N, multi_rows_per_block(m));
  int kc = (65536 / 4) / m;
  kc = (kc / 512) * 512;
  const int want_splits = ceil_div(512, row_blocks);
  int by_blocks = ceil_div(K, want_splits);
  by_blocks = ceil_div(by_blocks, 512) * 512;
  if (by_blocks < kc) kc = by_blocks;
  if (kc < 512) kc = 512;
  return kc;
}

int gemv_multi_splits(int rows, int N, int K) {
  const int m = gemv_multi_width(rows);
  if (m < 0) return -1;
  return ceil_div(K, multi_kchunk(m, N, K));
}

hipError_t launch_gemv_multi(const uint16_t* W, const uint16_t* S, int N, int K, const float* x0,
                             const float* x1, const float* x2, int seg, int rows, float* P,
                             int* splits_out, hipStream_t s, const TapRowsB& yb) {
  const int m = gemv_multi_width(rows);
  if (m < 0 || (K % (S ? 32 : 8)) || (x1 && (seg % 4))) return hipErrorInvalidValue;
  if (yb.rows_x < rows && (!x1 || !yb.y[0] || !yb.y[1] || !yb.y[2])) return hipErrorInvalidValue;
  const int kc = multi_kchunk(m, N, K);
  const int splits = ceil_div(K, kc);
  *splits_out = splits;
  dim3 grid(ceil_div(N, multi_rows_per_block(m)), splits), block(512);
  // the staged floats, and with int4 weights their digit planes and exponents
  const size_t lds = S ? size_t(m) * (2 * kc + kc / 2 + kc / 8) : size_t(m) * kc * sizeof(float);
  switch (m) {
#define MCASE(MM)                                                                              \
  case MM:                                                                                     \
    if (S) {                                                                                   \
      E3_LDS_ALLOW((k_gemv_multi<MM, true>), lds);                                             \
      hipLaunchKernelGGL((k_gemv_multi<MM, true>), grid, block, lds, s, W, S, N, K, kc, x0, x1, x2, \
                         seg, rows, P, yb);                                                    \
    } else                                                                                     \
      hipLaunchKernelGGL((k_gemv_multi<MM, false>), grid, block, lds, s, W, S, N, K, kc, x0, x1,  \
                         x2, seg, rows, P, yb);                                                \
    break;
    MCASE(1) MCASE(2) MCASE(3) MCASE(4) MCASE(5) MCASE(6) MCASE(8) MCASE(9) MCASE(12) MCASE(16)
#undef MCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// k_gemv_multi_qh with int4 weights: blocks [0, qb) the hidden-half sums (qh_i4_block in
// the int4 GEMVs' 8-wave, 2-row, 2-step form over nvq virtual blocks), the rest the
// int4 multi-vector GEMV's (row block, K chunk) grid
template <int M>
__global__ __launch_bounds__(512) void k_gemv_multi_qh_i4(const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ S, int N, int K, int kc,
                                                          const float* __restrict__ x0, int rows,
                                                          float* __restrict__ P, QhArgs q, int qb, int nvq, int gx) {
  static_assert(MultiShape<M>::WAVES == 8, "512 threads");
  extern __shared__ float xs[];
  __shared__ float red[32];
  const int b = int(blockIdx.x);
  if (b < qb) {
    qh_i4_block<8, 2, 2>(q, b, qb, nvq, xs, red);
    return;
  }
  const int t = b - qb;
  const TapRowsB none{{nullptr, nullptr, nullptr}, 1 << 30};
  gemv_multi_block<M, true>(t % gx, t / gx, W, S, N, K, kc, x0, nullptr, nullptr, 0, rows, P, none, xs);
}

hipError_t launch_gemv_multi_qh(const uint16_t* W, const uint16_t* S, int N, int K, const float* x0, int rows,
                                float* P, int* splits_out, const QhArgs& q, hipStream_t s) {
  const int m = gemv_multi_width(rows);
  if (S) {  // int4: W codes and S scales of the K/V rows, q the int4 hidden half
    if (m < 0 || (K % 32) || !q.s || (q.n % 32) || (q.k0 % 32) || q.N < 1) return hipErrorInvalidValue;
    const int kc = multi_kchunk(m, N, K);
    const int splits = ceil_div(K, kc);
    *splits_out = splits;
    const int gx = ceil_div(N, multi_rows_per_block(m)), nvq = ceil_div(q.N, 16), qb = i4_grid(nvq);
    const size_t lds = std::max(size_t(m) * (2 * kc + kc / 2 + kc / 8), size_t(q.n) * sizeof(float) + q_vec_bytes(q.n));
    switch (m) {
#define MCASE(MM)                                                                                        \
  case MM:                                                                                               \
    E3_LDS_ALLOW((k_gemv_multi_qh_i4<MM>), lds);                                                         \
    E3_LAUNCH((k_gemv_multi_qh_i4<MM>), dim3(qb + gx * splits), dim3(512), lds, s, W, S, N, K, kc, x0, rows, \
              P, q, qb, nvq, gx);                                                                        \
    break;
      MCASE(1) MCASE(2) MCASE(3) MCASE(4) MCASE(5) MCASE(6) MCASE(8) MCASE(9) MCASE(12) MCASE(16)
#undef MCASE
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (m < 0 || (K % 8) || q.s || (q.n % 8) || q.N < 1) return hipErrorInvalidValue;
  const int kc = multi_kchunk(m, N, K);
  const int splits = ceil_div(K, kc);
  *splits_out = splits;
  const int gx = ceil_div(N, multi_rows_per_block(m)), qb = ceil_div(q.N, 16);
  const size_t lds = std::max(size_t(m) * kc, size_t(q.n)) * sizeof(float);
  switch (m) {
#define MCASE(MM)                                                                                  \
  case MM:                                                                                         \
    E3_LDS_ALLOW((k_gemv_multi_qh<MM>), lds);                                                      \
    E3_LAUNCH((k_gemv_multi_qh<MM>), dim3(qb + gx * splits), dim3(512), lds, s, W, N, K, kc, x0, rows, P, q, \
              qb, gx);                                                                             \
    break;
    MCASE(1) MCASE(2) MCASE(3) MCASE(4) MCASE(5) MCASE(6) MCASE(8) MCASE(9) MCASE(12) MCASE(16)
#undef MCASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace e3
