// fp32 blockwise attention with online-softmax merge (fp32 throughout: no
// bf16 and no reduced-precision matrix path), for fp32 inputs.
//
// One thread owns one query row: its unnormalised output stays in registers
// and its Q row in LDS while the workgroup streams the KV blocks through LDS in tiles of
// BN keys.  Per tile the thread forms the tile's scores s_j = scale * <q, k_j>
// (natural-log units), masks keys that are past the block end or (causal)
// after the row, and folds them into its state with the exact online-softmax
// rule: m' = max(m, max_j s_j), alpha = exp(m - m'), l' = alpha*l + sum_j
// exp(s_j - m'), acc' = alpha*acc + sum_j exp(s_j - m') v_j.
// K/V reads from LDS are the same address for every lane (broadcast).
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kRows = 64;  // rows (threads) per workgroup
constexpr int BN = 16;     // keys per tile

__device__ __forceinline__ int tiles_for(const AttnArgs& a, int64_t pos0, int len, int64_t last_pos) {
  int64_t nk = len;
  if (a.causal) {
    const int64_t lim = last_pos - pos0 + 1;
    nk = lim < 0 ? 0 : (lim < nk ? lim : nk);
  }
  return (int)((nk + BN - 1) / BN);
}

template <int D, int MODE>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(AttnArgs a, BlockTable tbl) {
  __shared__ float qs[kRows][D + 1];  // +1: rows read by different lanes fall in different banks
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  const int n_qt = (int)((a.q_len + kRows - 1) / kRows);
  const int wid = blockIdx.x;
  const int bh = wid / n_qt;
  const int qt = n_qt - 1 - (wid - bh * n_qt);
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)qt * kRows;
  const int64_t r = row0 + tid;
  const bool row_ok = r < a.q_len;
  const int64_t my_pos = a.q_pos0 + r;
  const int64_t last_pos = a.q_pos0 + ((row0 + kRows < a.q_len) ? row0 + kRows : a.q_len) - 1;

  for (int e = tid; e < kRows * D; e += kRows) {
    const int rr = e / D, d = e % D;
    const int64_t row = row0 + rr;
    qs[rr][d] = row < a.q_len ? ((const float*)a.q)[b * a.q_sb + row * a.q_ss + h * a.q_sh + d] : 0.f;
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  const int64_t sidx = ((int64_t)b * a.heads + h) * a.q_len + r;
  float m = -INFINITY, l = 0.f;
  if ((MODE == kLoadStore || MODE == kLoadFinalize) && row_ok) {
    m = a.m[sidx];
    l = a.l[sidx];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = a.acc[sidx * D + d];
  }

  auto score = [&](int j) -> float {
    float dot = 0.f;
#pragma unroll 16
    for (int d = 0; d < D; ++d) dot = __builtin_fmaf(qs[tid][d], ks[j][d], dot);
    return dot * a.scale;
  };

  for (int bi = 0; bi < a.nblocks; ++bi) {
    const int64_t pos0 = tbl.pos0[bi];
    const int64_t len = tbl.len[bi];  // valid keys of the block
    const int nt = tiles_for(a, pos0, (int)len, last_pos);
    const float* kb = (const float*)tbl.k[bi] + b * a.kv_sb + h * a.kv_sh;
    const float* vb = (const float*)tbl.v[bi] + b * a.kv_sb + h * a.kv_sh;
    for (int t = 0; t < nt; ++t) {
      __syncthreads();
      for (int e = tid; e < BN * D; e += kRows) {
        const int j = e / D, d = e % D;
        const int64_t kk = (int64_t)t * BN + j;
        ks[j][d] = kk < len ? kb[kk * a.kv_ss + d] : 0.f;
        vs[j][d] = kk < len ? vb[kk * a.kv_ss + d] : 0.f;
      }
      __syncthreads();
      // pass 1: the tile's largest visible score
      int nlive = 0;
      float mt = -INFINITY;
#pragma unroll 1
      for (int j = 0; j < BN; ++j) {
        const int64_t kk = (int64_t)t * BN + j;
        if (kk < len && (!a.causal || pos0 + kk <= my_pos)) {
          mt = fmaxf(mt, score(j));
          ++nlive;
        }
      }
      if (nlive == 0) continue;  // nothing visible in this tile for this row
      // rescale the carried state to the new running max, then accumulate
      const float m_new = fmaxf(m, mt);
      const float alpha = expf(m - m_new);  // 0 when m = -inf
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll 1
      for (int j = 0; j < BN; ++j) {
        const int64_t kk = (int64_t)t * BN + j;
        if (kk < len && (!a.causal || pos0 + kk <= my_pos)) {
          const float p = expf(score(j) - m_new);
          l += p;
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vs[j][d], acc[d]);
        }
      }
      m = m_new;
    }
  }

  if (!row_ok) return;
  if (MODE == kInitStore || MODE == kLoadStore) {
    a.m[sidx] = m;
    a.l[sidx] = l;
#pragma unroll
    for (int d = 0; d < D; ++d) a.acc[sidx * D + d] = acc[d];
  } else {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    a.lse[sidx] = l > 0.f ? m + logf(l) : -INFINITY;
    float* op = (float*)a.o + b * a.o_sb + r * a.o_ss + h * a.o_sh;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  }
}

template <int D, int MODE>
hipError_t launch_t(const AttnArgs& a, const BlockTable& t, hipStream_t s) {
  const int64_t n_qt = (a.q_len + kRows - 1) / kRows;
  const int64_t n_work = (int64_t)a.batch * a.heads * n_qt;
  if (n_work == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_f32_kernel<D, MODE>), dim3((unsigned)n_work), dim3(kRows), 0, s, a, t);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mode(const AttnArgs& a, const BlockTable& t, int mode, hipStream_t s) {
  switch (mode) {
    case kInitFinalize: return launch_t<D, kInitFinalize>(a, t, s);
    case kInitStore: return launch_t<D, kInitStore>(a, t, s);
    case kLoadStore: return launch_t<D, kLoadStore>(a, t, s);
    default: return launch_t<D, kLoadFinalize>(a, t, s);
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, const BlockTable& t, int mode, hipStream_t s) {
  return a.head_dim == 128 ? launch_mode<128>(a, t, mode, s) : launch_mode<64>(a, t, mode, s);
}

}  // namespace ra
