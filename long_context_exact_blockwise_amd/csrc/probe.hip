// Measurement helper: bf16 MFMA throughput probe, gfx950.
//
// Every wave issues back-to-back independent v_mfma_f32_32x32x16_bf16 (four
// accumulator chains, no memory traffic in the loop), so the matrix cores of
// every SIMD the grid occupies stay busy for the whole launch.  Timed on the
// host, it gives the bf16 MFMA rate the part sustains under load (its clock
// under that power draw), the reference against which the attention and
// feedforward kernels' MFMA fractions are read beside the published peak.
#include "attn_common.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kProbeThreads = 512;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 x, y;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
    y[j] = (__bf16)(0.002f * (float)((lane * 3 + j) & 7));
  }
  f32x16 a0 = f32x16{}, a1 = f32x16{}, a2 = f32x16{}, a3 = f32x16{};
  for (int i = 0; i < iters; ++i) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, x, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, y, a3, 0, 0, 0);
  }
  // keep the products live: one value per thread
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = a0[0] + a1[5] + a2[10] + a3[15];
}

}  // namespace

hipError_t launch_probe_mfma(float* out, int workgroups, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace ra
