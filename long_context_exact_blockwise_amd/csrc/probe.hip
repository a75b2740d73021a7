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
// holds, depends on the operand bits.  A third form reads one operand of
// every product from LDS at a set ratio of LDS bytes per product.
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

// The same products with each one's A operand read from LDS: per iteration a
// wave reads NR 16-byte fragments (64 lanes x 16 bytes, 1 KiB each) from a
// 64 KiB LDS image of the workgroup's operands and issues 16 products, each
// fragment feeding 16 / NR of them, so a wave reads NR / 16 KiB of LDS per
// product (NR = 16: 1 KiB per 32x32x16 product).  The read windows rotate
// with the iteration so that no read can be hoisted out of the loop.  It
// measures the bf16 MFMA rate the part holds while the LDS traffic of a
// kernel that reads every operand fragment once per product draws power
// beside the matrix cores.
template <int NR>
__global__ __launch_bounds__(kProbeThreads) void mfma_lds_probe_kernel(const bf16x8* src, float* out, int iters) {
  static_assert(16 % NR == 0, "each fragment feeds 16 / NR products");
  __shared__ __attribute__((aligned(16))) bf16x8 img[4096];  // 64 KiB
  const bf16x8* wsrc = src + (int64_t)blockIdx.x * kProbeThreads * 4;  // this workgroup's 2048 fragments
  for (int i = threadIdx.x; i < 4096; i += kProbeThreads) img[i] = wsrc[i & 2047];
  __syncthreads();
  const bf16x8* s4 = wsrc + threadIdx.x * 4;
  const bf16x8 b0 = s4[0], b1 = s4[1], b2 = s4[2], b3 = s4[3];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t base = lds_addr_of((const char*)img);
  f32x16 a0 = f32x16{}, a1 = f32x16{}, a2 = f32x16{}, a3 = f32x16{};
  for (int it = 0; it < iters; ++it) {
    const uint32_t wb = (uint32_t)((wave * 8 + (it & 7)) & 63) << 10;
    bf16x8 fr[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) fr[j] = *(lds_bf16x8*)(size_t)(base + ((wb + j * 1024 + lane * 16) & 0xFFFFu));
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(j + 0) % NR], b0, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(j + 1) % NR], b1, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(j + 2) % NR], b2, a2, 0, 0, 0);
      a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(j + 3) % NR], b3, a3, 0, 0, 0);
    }
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = a0[0] + a1[5] + a2[10] + a3[15];
}

}  // namespace

hipError_t launch_probe_mfma_lds(const void* src, float* out, int workgroups, int iters, int lds_reads,
                                 hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(kProbeThreads);
  const bf16x8* b = (const bf16x8*)src;
  if (lds_reads == 4)
    hipLaunchKernelGGL(mfma_lds_probe_kernel<4>, grid, block, 0, s, b, out, iters);
  else if (lds_reads == 8)
    hipLaunchKernelGGL(mfma_lds_probe_kernel<8>, grid, block, 0, s, b, out, iters);
  else
    hipLaunchKernelGGL(mfma_lds_probe_kernel<16>, grid, block, 0, s, b, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(const void* src, float* out, int workgroups, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, (const bf16x8*)src, out,
                     iters);
  return hipGetLastError();
}

}  // namespace ra
