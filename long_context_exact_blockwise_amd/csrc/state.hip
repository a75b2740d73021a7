// State kernels of the per-block ring pass: start (m = -inf, l = 0, acc = 0)
// and finish (O = acc / l, LSE = m + ln l) the online-softmax triple of the
// "Gotchas and Failure Modes" section of "Ring Attention: Train 1M Tokens on
// 8GB GPUs in 2026"; plus a plain copy kernel used as a byte-counter and
// bandwidth reference.  All three are HBM-bound streaming kernels: 16-byte
// accesses, consecutive lanes on consecutive addresses.
#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void init_state_kernel(int64_t rows, int32_t d4, float* m, float* l,
                                                              float* acc) {
  const int64_t n = rows * d4;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    ((f32x4*)acc)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < rows) {
      m[i] = -INFINITY;
      l[i] = 0.f;
    }
  }
}

// One thread per (row, 4 consecutive d): rows are (b, h, r) in state order.
template <typename OutT>
__global__ __launch_bounds__(kThreads) void finalize_kernel(AttnArgs a) {
  const int d4n = a.head_dim / 4;
  const int64_t n = (int64_t)a.batch * a.heads * a.q_len * d4n;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / d4n;
    const int d4 = (int)(i - row * d4n);
    const int64_t bh = row / a.q_len;
    const int64_t r = row - bh * a.q_len;
    const int64_t b = bh / a.heads;
    const int64_t h = bh - b * a.heads;
    const float lv = a.l[row];
    const float inv = lv > 0.f ? 1.0f / lv : 0.f;
    const f32x4 v = ((const f32x4*)a.acc)[i];
    OutT* op = (OutT*)a.o + b * a.o_sb + r * a.o_ss + h * a.o_sh + 4 * d4;
    if constexpr (sizeof(OutT) == 2) {
      bf16x4 o4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o4[j] = (__bf16)(v[j] * inv);
      *(bf16x4*)op = o4;
    } else {
      *(f32x4*)op = f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
    }
    if (d4 == 0) a.lse[row] = lv > 0.f ? a.m[row] + logf(lv) : -INFINITY;
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

// Backward preprocessing: delta[row] = sum_d dO[row, d] O[row, d] (rows in
// state order (b, h, r)).  D/8 consecutive lanes share a row, 8 elements
// (16 bytes of dO) each, and reduce with lane swaps.
template <typename OutT>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(AttnArgs a, const __bf16* __restrict__ dout,
                                                             float* __restrict__ delta) {
  const int tpr = a.head_dim / 8;
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = g / tpr;
  const int part = (int)(g - row * tpr);
  const int64_t nrow = (int64_t)a.batch * a.heads * a.q_len;
  float sum = 0.f;
  if (row < nrow) {
    const int64_t bh = row / a.q_len;
    const int64_t r = row - bh * a.q_len;
    const int64_t b = bh / a.heads;
    const int64_t h = bh - b * a.heads;
    const __bf16* dp = dout + b * a.q_sb + r * a.q_ss + h * a.q_sh + 8 * part;
    const OutT* op = (const OutT*)a.o + b * a.o_sb + r * a.o_ss + h * a.o_sh + 8 * part;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += (float)dp[j] * (float)op[j];
  }
  for (int m = 1; m < tpr; m <<= 1) sum += __shfl_xor(sum, m);
  if (row < nrow && part == 0) delta[row] = sum;
}

// n 32-bit words set to `value` (0 is +0.0f; all ones is a NaN both as one
// fp32 and as two bf16 values).
__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    p[i] = value;
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 16;  // 16 workgroups per CU, grid-stride beyond
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_init_state(int64_t rows, int32_t d, float* m, float* l, float* acc, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t n = rows * (d / 4);
  hipLaunchKernelGGL(init_state_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, rows, d / 4, m, l, acc);
  return hipGetLastError();
}

hipError_t launch_finalize(const AttnArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.batch * a.heads * a.q_len * (a.head_dim / 4);
  if (n == 0) return hipSuccess;
  if (a.out_bf16)
    hipLaunchKernelGGL(finalize_kernel<__bf16>, dim3(grid_for(n)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, dim3(grid_for(n)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, (const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const AttnArgs& a, const void* dout, float* delta, hipStream_t s) {
  const int64_t n = (int64_t)a.batch * a.heads * a.q_len * (a.head_dim / 8);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
  if (a.out_bf16)
    hipLaunchKernelGGL(bwd_delta_kernel<__bf16>, dim3(grid), dim3(kThreads), 0, s, a, (const __bf16*)dout, delta);
  else
    hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3(grid), dim3(kThreads), 0, s, a, (const __bf16*)dout, delta);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, hipStream_t s) { return launch_fill_u32(p, n, 0u, s); }

hipError_t launch_fill_u32(void* p, int64_t n, uint32_t value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, (uint32_t*)p, n, value);
  return hipGetLastError();
}

}  // namespace ra
