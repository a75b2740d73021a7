// Measurement helper: bf16 MFMA throughput probe, gfx950.
//
// Every wave issues back-to-back independent v_mfma_f32_32x32x16_bf16 (four
// accumulator chains, no memory traffic in the loop), so the matrix cores of
// every SIMD the grid occupies stay busy for the whole launch.  Timed on the
// host, it gives the bf16 MFMA rate the part sustains under load (its clock
// under that power draw), the reference against which the attention and
// feedforward kernels' MFMA fractions are read beside the published peak.
// The operands are either a fixed pattern of small values (few bits toggle
// between products) or four fragments per thread read once from a caller
// buffer, e.g. random bf16 values: the power drawn, hence the clock the part
// holds, depends on the operand bits.
#include "attn_common.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kProbeThreads = 512;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(const bf16x8* src, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 x, y, x2, y2;
  if (src) {
    const bf16x8* s4 = src + ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) * 4;
    x = s4[0];
    y = s4[1];
    x2 = s4[2];
    y2 = s4[3];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
      y[j] = (__bf16)(0.002f * (float)((lane * 3 + j) & 7));
    }
    x2 = y;
    y2 = x;
  }
  f32x16 a0 = f32x16{}, a1 = f32x16{}, a2 = f32x16{}, a3 = f32x16{};
  for (int i = 0; i < iters; ++i) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x2, y, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y2, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x2, y2, a3, 0, 0, 0);
  }
  // keep the products live: one value per thread
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = a0[0] + a1[5] + a2[10] + a3[15];
}

}  // namespace

hipError_t launch_probe_mfma(const void* src, float* out, int workgroups, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, (const bf16x8*)src, out,
                     iters);
  return hipGetLastError();
}

}  // namespace ra
