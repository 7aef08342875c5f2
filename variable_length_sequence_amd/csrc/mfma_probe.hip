// Matrix-core throughput probe: every wave issues long runs of independent
// 32x32x16 bf16 MFMAs from registers (no memory traffic in the loop), so the
// measured rate is what the matrix cores sustain under full load at the clock
// the chip holds, the reachable ceiling for the attention kernels.
#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kChains = 8;   // independent accumulators per wave

__global__ void __launch_bounds__(kProbeThreads)
mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float((lane + i) & 7) * 0.125f);
    b[i] = (__bf16)(float((lane * 3 + i) & 7) * 0.0625f);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

int64_t mfma_probe_flops(int32_t iters, int32_t n_wg) {
  return int64_t(n_wg) * (kProbeThreads / 64) * iters * kChains * (2LL * 32 * 32 * 16);
}

hipError_t launch_mfma_probe(int32_t iters, int32_t n_wg, float* sink, hipStream_t stream) {
  ProfScope prof("mfma_probe", stream);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_wg), dim3(kProbeThreads), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace vl
