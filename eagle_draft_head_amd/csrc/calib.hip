// Calibration of the two ceilings the kernels are measured against, on the GPU at
// hand (clocks under load, fabric limits):
//   * the bf16 MFMA rate it sustains: every wave runs four independent chains of
//     v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic (the
//     loop compiles to the four MFMAs and the counter; with the 16x16x32 form the
//     compiler copies accumulators between the MFMAs);
//   * its streaming HBM read rate: the weight stream's access pattern -- each wave
//     reads contiguous 16 KB runs, a non-temporal 16-byte load per lane, four loads
//     in flight per lane -- over a buffer read right after another buffer larger than
//     the infinity cache, so the measured buffer comes from HBM.
// Each is timed with HIP events over single launches, the best of several.
#include <hip/hip_runtime.h>

#include "../../include/eagle3.h"
#include "common.hpp"

namespace e3 {

typedef __bf16 cal_bf16x8 __attribute__((ext_vector_type(8)));
typedef float cal_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCalChains = 4;
constexpr int kCalBlocks = 2048;  // 8 blocks of 4 waves per CU
constexpr int kCalThreads = 256;

__global__ __launch_bounds__(kCalThreads) void k_calib_mfma(int iters, float* __restrict__ out) {
  cal_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float(int(threadIdx.x & 15) + i) * 0.0625f);
    b[i] = (__bf16)(float(i - int(threadIdx.x & 7)) * 0.03125f);
  }
  cal_f32x16 c0{}, c1{}, c2{}, c3{};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const cal_f32x16 t = (c0 + c1) + (c2 + c3);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += t[i];
  if (s == 1.2345e30f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the chains
}

constexpr int kCalRun16 = 1024;  // 16-byte chunks of a wave's contiguous run (16 KB)
constexpr int kCalReadU = 4;

// waves take runs w, w + (waves in the grid), ...; the last run may be short (loads
// are clamped to it)
__global__ __launch_bounds__(kCalThreads) void k_calib_read(const uint4* __restrict__ p, size_t n16,
                                                            uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (kCalThreads / 64) + (threadIdx.x >> 6);
  const size_t waves = (size_t)gridDim.x * (kCalThreads / 64);
  const size_t runs = (n16 + kCalRun16 - 1) / kCalRun16;
  for (size_t r = wave; r < runs; r += waves) {
    const uint4* q = p + r * kCalRun16;
    const int len = int(min<size_t>(kCalRun16, n16 - r * kCalRun16));
    for (int j = lane; j < len; j += 64 * kCalReadU) {
      uint4 v[kCalReadU];
#pragma unroll
      for (int u = 0; u < kCalReadU; ++u) v[u] = ld_stream(q + min(j + 64 * u, len - 1));
#pragma unroll
      for (int u = 0; u < kCalReadU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;  // keeps the loads
}

}  // namespace e3

namespace {

// best (shortest) of reps timed launches, in ms
template <typename Launch>
int best_ms(int reps, hipStream_t s, Launch launch, float* best) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return EAGLE3_E_HIP;
  if (hipEventCreate(&e1) != hipSuccess) { (void)hipEventDestroy(e0); return EAGLE3_E_HIP; }
  int rc = EAGLE3_OK;
  *best = 0.f;
  for (int r = 0; r < reps && rc == EAGLE3_OK; ++r) {
    hipError_t e = launch(true);
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    if (e == hipSuccess) e = launch(false);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess) rc = EAGLE3_E_HIP;
    else if (r == 0 || ms < *best) *best = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

}  // namespace

extern "C" {

int eagle3_calibrate_mfma(int32_t iters, int32_t reps, float* sink_dev, double* tflops, void* stream) {
  if (iters < 1 || reps < 1 || !sink_dev || !tflops) return EAGLE3_E_INVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float ms = 0.f;
  const int rc = best_ms(reps, s, [&](bool warm) {
    hipLaunchKernelGGL(e3::k_calib_mfma, dim3(e3::kCalBlocks), dim3(e3::kCalThreads), 0, s,
                       warm ? 1 : iters, sink_dev);
    return hipGetLastError();
  }, &ms);
  if (rc) return rc;
  const double flops = double(e3::kCalBlocks) * (e3::kCalThreads / 64) * double(iters) * e3::kCalChains *
                       (2.0 * 32 * 32 * 16);
  *tflops = flops / (double(ms) * 1e-3) / 1e12;
  return EAGLE3_OK;
}

int eagle3_calibrate_stream(const void* buf_dev, size_t bytes, const void* flush_dev, size_t flush_bytes,
                            int32_t reps, uint32_t* sink_dev, double* gbs, void* stream) {
  if (!buf_dev || !flush_dev || !sink_dev || !gbs || reps < 1 || bytes < 16 || flush_bytes < 16)
    return EAGLE3_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(buf_dev) | reinterpret_cast<uintptr_t>(flush_dev)) & 15u)
    return EAGLE3_E_INVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float ms = 0.f;
  const int rc = best_ms(reps, s, [&](bool flush) {
    const void* p = flush ? flush_dev : buf_dev;
    const size_t n16 = (flush ? flush_bytes : bytes) / 16;
    hipLaunchKernelGGL(e3::k_calib_read, dim3(e3::kCalBlocks), dim3(e3::kCalThreads), 0, s,
                       static_cast<const uint4*>(p), n16, sink_dev);
    return hipGetLastError();
  }, &ms);
  if (rc) return rc;
  *gbs = double(bytes / 16 * 16) / (double(ms) * 1e-3) / 1e9;
  return EAGLE3_OK;
}

}  // extern "C"
