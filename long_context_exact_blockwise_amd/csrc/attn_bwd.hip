// Backward of blockwise attention for one KV block, bf16 inputs, gfx950.
//
// The pages train through the ring ("Ring Attention: Train 1M Tokens on 8GB
// GPUs in 2026", sections "Training Speed: The Numbers" and "Gotchas and
// Failure Modes": gradients flow backwards through the ring) without writing
// the backward out; these kernels compute the exact gradient of the exact
// forward.  With P = exp(scale q.k - LSE) (the forward's LSE, so no max or sum
// is recomputed), dP = dO . v and delta = <dO, O> per row:
//   dS = P (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// A device computes dQ of its chunk (summed over the blocks) and, for each
// block it receives, its contribution to that block's dK and dV, which in the
// ring travel on with the block.  All three are accumulated (+=) in fp32.
//
// Two kernels per block:
//   dq kernel:   a workgroup owns query rows and streams the block's key tiles
//                (the forward's structure): S^T = K Q^T, dP^T = V dO^T, then
//                dQ^T += K^T dS^T.  Q and dO fragments stay in registers.
//   dkdv kernel: a workgroup owns keys (K, V fragments in registers) and
//                streams query tiles: S = Q K^T, dP = dO V^T, then
//                dV^T += dO^T P and dK^T += Q^T dS.
// Matrix products use v_mfma_f32_32x32x16_bf16 with the same operand layouts
// as the forward kernel: transposed-operand fragments (K^T, dO^T, Q^T) come
// from LDS with ds_read_b64_tr_b16 in the 4-row-group key order that matches
// the accumulator layout of the score fragments.
#include "attn_common.h"
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int kBWaves = 4;                 // waves per workgroup in both kernels
constexpr int kBThreads = 64 * kBWaves;
constexpr int BQ = 32 * kBWaves;           // dq kernel: query rows per workgroup
constexpr int BKN = 64;                    // dq kernel: keys per tile
constexpr int BKK = 32 * kBWaves;          // dkdv kernel: keys per workgroup
constexpr int BQT = 32;                    // dkdv kernel: query rows per tile

template <int D>
struct BCfg {
  static constexpr int CH = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int KT = BKN * ROWB;  // bytes of a 64-key tile
  static constexpr int QT = BQT * ROWB;  // bytes of a 32-row tile
  static constexpr int DQ_LDS = 2 * 3 * KT;   // two buffers of (K rows, K transposed reads, V rows)
  static constexpr int DKDV_LDS = 2 * 4 * QT;  // two buffers of (Q, Q transposed, dO, dO transposed)
};

// Copy rows 0..nrows-1 of a row-major bf16 tile (row r at src + r*row_bytes)
// into LDS at dst, chunk placement swizzled for row reads (VSWZ false, as
// k_off) or for transpose reads (VSWZ true, as v_off).  Rows at or past
// `valid` re-read row valid-1 (their values are masked out).  The copies of
// the workgroup are shared out over its waves; wait with vmcnt before use.
template <int D, bool VSWZ>
__device__ __forceinline__ void copy_tile(const char* src, int64_t row_bytes, int valid, uint32_t dst, int nrows,
                                          int wave, int lane) {
  const int nchunks = nrows * D * 2 / 1024;
  for (int c = wave; c < nchunks; c += kBWaves) {
    const int p = c * 1024 + lane * 16;
    const int row = p / (D * 2);
    const int cs = (p % (D * 2)) / 16;
    const int col = (VSWZ ? v_off<D>(row, cs) : k_off<D>(row, cs)) / 16 - row * (D / 8);  // XOR is self-inverse
    const int rr = row < valid ? row : valid - 1;
    lds_dma16(src, (uint32_t)(rr * row_bytes + col * 16), dst + c * 1024);
  }
}

// Transpose-read fragment (the A operand of a product whose contraction runs
// over tile rows): rows `row` + {key0, key0 + 8} (+0..3 across lane groups),
// columns 32 db + ..., exactly as the forward kernel gathers V^T.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(uint32_t tile, int vA, int db, int row) {
  const uint32_t va = tile + (vA ^ (64 * db)) + row * (D * 2);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)va);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(va + 8 * D * 2));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane base offset of tr_frag (lane 4t+s of 16-lane group g addresses row
// t of a 4-row group, columns 4s..4s+3 of a 16-column slice).
template <int D>
__device__ __forceinline__ int tr_base(int lane) {
  const int g4 = lane >> 4;
  const int tr_t = (lane >> 2) & 3;
  const int tr_s = lane & 3;
  const int key0 = 4 * (g4 >> 1) + tr_t;
  return v_off<D>(key0, 2 * (g4 & 1) + (tr_s >> 1)) + (tr_s & 1) * 8;
}

// Row of element i of a 32x32 MFMA result held by a lane in half hf.
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + (i & 3) + 4 * hf; }

// ---------------------------------------------------------------------------
// dQ: one workgroup per BQ query rows of one (b, h); this lane's row r.
template <int D>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using C = BCfg<D>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int n_qt = (int)((a.q_len + BQ - 1) / BQ);
  const int n_work = a.batch * a.heads * n_qt;
  const int per = (n_work + 7) >> 3;
  const int wid = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (wid >= n_work) return;
  const int bh = wid / n_qt;
  const int qt = n_qt - 1 - (wid - bh * n_qt);
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int64_t row0 = (int64_t)qt * BQ;
  const int64_t r = row0 + 32 * wave + l32;
  const bool row_ok = r < a.q_len;
  const int64_t q_last = a.q_pos0 + ((row0 + BQ < a.q_len) ? row0 + BQ : a.q_len) - 1;
  int64_t nk = a.kv_len;
  if (a.causal) {
    const int64_t lim = q_last - a.kv_pos0 + 1;
    nk = lim < 0 ? 0 : (lim < nk ? lim : nk);
  }
  const int n_tiles = (int)((nk + BKN - 1) / BKN);
  if (n_tiles == 0) return;

  bf16x8 qf[C::KS], df[C::KS];
  {
    const int64_t off = b * a.q_sb + r * a.q_ss + h * a.q_sh + 8 * hf;
    const __bf16* qp = (const __bf16*)a.q + off;
    const __bf16* dp = (const __bf16*)a.dout + off;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (row_ok) {
        qf[ks] = *(const bf16x8*)(qp + 16 * ks);
        df[ks] = *(const bf16x8*)(dp + 16 * ks);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[ks][j] = df[ks][j] = (__bf16)0.0f;
      }
    }
  }
  const int64_t sidx = ((int64_t)b * a.heads + h) * a.q_len + (row_ok ? r : 0);
  const float lse_r = a.lse[sidx];
  const bool row_live = row_ok && lse_r > -INFINITY;  // a row that saw no key anywhere has no gradient
  const float lse2 = row_live ? lse_r * kLog2e : 0.f;
  const float dlt = row_live ? a.delta[sidx] : 0.f;
  const float c2 = a.scale * kLog2e;
  const int64_t my_pos = a.q_pos0 + r;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  const uint32_t base = lds_addr_of(lds);
  const int64_t row_bytes = a.kv_ss * 2;
  const char* ksrc = (const char*)a.k + (b * a.kv_sb + h * a.kv_sh) * 2;
  const char* vsrc = (const char*)a.v + (b * a.kv_sb + h * a.kv_sh) * 2;
  auto issue = [&](int t, int buf) {
    const int64_t go = (int64_t)t * BKN * row_bytes;
    const int valid = (int)(a.kv_len - (int64_t)t * BKN);
    const uint32_t dst = base + buf * 3 * C::KT;
    copy_tile<D, false>(ksrc + go, row_bytes, valid, dst, BKN, wave, lane);
    copy_tile<D, true>(ksrc + go, row_bytes, valid, dst + C::KT, BKN, wave, lane);
    copy_tile<D, false>(vsrc + go, row_bytes, valid, dst + 2 * C::KT, BKN, wave, lane);
  };
  const int vA = tr_base<D>(lane);

  issue(0, 0);
  wait_vm<0>();
  wg_barrier();
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) issue(t + 1, (t + 1) & 1);
    const uint32_t kl = base + (t & 1) * 3 * C::KT;
    const uint32_t ktl = kl + C::KT;
    const uint32_t vl = kl + 2 * C::KT;
    // S^T = K Q^T and dP^T = V dO^T (rows: 64 keys in two 32-key halves kb)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int o = k_off<D>(l32 + 32 * kb, 2 * ks + hf);
        const bf16x8 kf = *(lds_bf16x8*)(size_t)(kl + o);
        const bf16x8 vf = *(lds_bf16x8*)(size_t)(vl + o);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[ks], ks == 0 ? f32x16{} : dp[kb], 0, 0, 0);
      }
    // dS^T = P^T (dP^T - delta), P^T = exp2(S^T c - LSE2); packed to bf16 pairs
    bf16x2 dsp[16];
    const int64_t key_t0 = (int64_t)t * BKN;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float v2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * q + u;
        const int kb = e >> 4, i = e & 15;
        const int64_t key = key_t0 + 32 * kb + acc_row(i, hf);
        const bool vis = row_live && key < a.kv_len && (!a.causal || a.kv_pos0 + key <= my_pos);
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c2, -lse2)) : 0.f;
        v2[u] = p * (dp[kb][i] - dlt);
      }
      dsp[q] = bf16x2{(__bf16)v2[0], (__bf16)v2[1]};
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const int q0 = 8 * kb + 4 * tp;
        const bf16x4 lo = __builtin_shufflevector(dsp[q0], dsp[q0 + 1], 0, 1, 2, 3);
        const bf16x4 hi = __builtin_shufflevector(dsp[q0 + 2], dsp[q0 + 3], 0, 1, 2, 3);
        const bf16x8 pf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(ktl, vA, db, 32 * kb + 16 * tp), pf, acc[db],
                                                            0, 0, 0);
      }
    wait_vm<0>();
    wg_barrier();
  }
  if (!row_ok) return;
  float* dq = a.dq + (((int64_t)b * a.q_len + r) * a.heads + h) * D + 4 * hf;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v4 = *(f32x4*)(dq + 32 * db + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] += a.scale * acc[db][4 * g + j];
      *(f32x4*)(dq + 32 * db + 8 * g) = v4;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per BKK keys of one (b, h); this lane's key c (as the
// column of the 32x32 products).
template <int D>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BCfg<D>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int n_kt = (int)((a.kv_len + BKK - 1) / BKK);
  const int n_work = a.batch * a.heads * n_kt;
  const int per = (n_work + 7) >> 3;
  const int wid = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (wid >= n_work) return;
  const int bh = wid / n_kt;
  const int kt = wid - bh * n_kt;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int64_t k0 = (int64_t)kt * BKK;
  const int64_t c = k0 + 32 * wave + l32;
  const bool key_ok = c < a.kv_len;
  // first query row that can see the workgroup's first key
  int64_t r_min = 0;
  if (a.causal) {
    r_min = a.kv_pos0 + k0 - a.q_pos0;
    if (r_min < 0) r_min = 0;
    if (r_min >= a.q_len) return;
  }
  const int n_qt = (int)((a.q_len + BQT - 1) / BQT);
  const int qt0 = (int)(r_min / BQT);

  bf16x8 kfr[C::KS], vfr[C::KS];
  {
    const int64_t off = b * a.kv_sb + c * a.kv_ss + h * a.kv_sh + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (key_ok) {
        kfr[ks] = *(const bf16x8*)((const __bf16*)a.k + off + 16 * ks);
        vfr[ks] = *(const bf16x8*)((const __bf16*)a.v + off + 16 * ks);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) kfr[ks][j] = vfr[ks][j] = (__bf16)0.0f;
      }
    }
  }
  const float c2 = a.scale * kLog2e;
  const int64_t key_pos = a.kv_pos0 + c;
  f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dk[db] = dv[db] = f32x16{};

  const uint32_t base = lds_addr_of(lds);
  const int64_t qrow_bytes = a.q_ss * 2;
  const char* qsrc = (const char*)a.q + (b * a.q_sb + h * a.q_sh) * 2;
  const char* osrc = (const char*)a.dout + (b * a.q_sb + h * a.q_sh) * 2;
  const float* lse_bh = a.lse + ((int64_t)b * a.heads + h) * a.q_len;
  const float* dl_bh = a.delta + ((int64_t)b * a.heads + h) * a.q_len;
  auto issue = [&](int t, int buf) {
    const int64_t go = (int64_t)t * BQT * qrow_bytes;
    const int valid = (int)(a.q_len - (int64_t)t * BQT);
    const uint32_t dst = base + buf * 4 * C::QT;
    copy_tile<D, false>(qsrc + go, qrow_bytes, valid, dst, BQT, wave, lane);
    copy_tile<D, true>(qsrc + go, qrow_bytes, valid, dst + C::QT, BQT, wave, lane);
    copy_tile<D, false>(osrc + go, qrow_bytes, valid, dst + 2 * C::QT, BQT, wave, lane);
    copy_tile<D, true>(osrc + go, qrow_bytes, valid, dst + 3 * C::QT, BQT, wave, lane);
  };
  const int vA = tr_base<D>(lane);

  issue(qt0, qt0 & 1);
  wait_vm<0>();
  wg_barrier();
  for (int t = qt0; t < n_qt; ++t) {
    if (t + 1 < n_qt) issue(t + 1, (t + 1) & 1);
    const uint32_t ql = base + (t & 1) * 4 * C::QT;
    const uint32_t qtl = ql + C::QT;
    const uint32_t ol = ql + 2 * C::QT;
    const uint32_t otl = ql + 3 * C::QT;
    // S = Q K^T and dP = dO V^T (rows: the tile's 32 queries; columns: keys)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int o = k_off<D>(l32, 2 * ks + hf);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(lds_bf16x8*)(size_t)(ql + o), kfr[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(lds_bf16x8*)(size_t)(ol + o), vfr[ks], dp, 0, 0, 0);
    }
    // P = exp2(S c - LSE2[row]), dS = P (dP - delta[row]); bf16 pairs of
    // consecutive elements (rows 8 (i>>2) + (i&3) + 4 hf)
    bf16x2 pp[8], dsp[8];
    const int64_t row_t0 = (int64_t)t * BQT;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float pv[2], dv2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 2 * q + u;
        const int64_t row = row_t0 + acc_row(i, hf);
        const int64_t rc = row < a.q_len ? row : a.q_len - 1;
        const float lse_r = lse_bh[rc];
        const bool vis = key_ok && row < a.q_len && lse_r > -INFINITY &&
                         (!a.causal || key_pos <= a.q_pos0 + row);
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -lse_r * kLog2e)) : 0.f;
        pv[u] = p;
        dv2[u] = p * (dp[i] - (vis ? dl_bh[rc] : 0.f));
      }
      pp[q] = bf16x2{(__bf16)pv[0], (__bf16)pv[1]};
      dsp[q] = bf16x2{(__bf16)dv2[0], (__bf16)dv2[1]};
    }
    // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 32 rows in two
    // 16-row steps tp)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const bf16x4 plo = __builtin_shufflevector(pp[4 * tp], pp[4 * tp + 1], 0, 1, 2, 3);
      const bf16x4 phi = __builtin_shufflevector(pp[4 * tp + 2], pp[4 * tp + 3], 0, 1, 2, 3);
      const bf16x8 pf = __builtin_shufflevector(plo, phi, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x4 slo = __builtin_shufflevector(dsp[4 * tp], dsp[4 * tp + 1], 0, 1, 2, 3);
      const bf16x4 shi = __builtin_shufflevector(dsp[4 * tp + 2], dsp[4 * tp + 3], 0, 1, 2, 3);
      const bf16x8 sf = __builtin_shufflevector(slo, shi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(otl, vA, db, 16 * tp), pf, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qtl, vA, db, 16 * tp), sf, dk[db], 0, 0, 0);
      }
    }
    wait_vm<0>();
    wg_barrier();
  }
  if (!key_ok) return;
  const int64_t o = (((int64_t)b * a.kv_cap + c) * a.heads + h) * D + 4 * hf;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 k4 = *(f32x4*)(a.dk + o + 32 * db + 8 * g);
      f32x4 v4 = *(f32x4*)(a.dv + o + 32 * db + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        k4[j] += a.scale * dk[db][4 * g + j];
        v4[j] += dv[db][4 * g + j];
      }
      *(f32x4*)(a.dk + o + 32 * db + 8 * g) = k4;
      *(f32x4*)(a.dv + o + 32 * db + 8 * g) = v4;
    }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  using C = BCfg<D>;
  static bool attr_done = false;  // set once per instantiation; the attribute is idempotent
  if (!attr_done) {
    hipError_t e =
        hipFuncSetAttribute((const void*)bwd_dq_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, C::DQ_LDS);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            C::DKDV_LDS);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t nq = (int64_t)a.batch * a.heads * ((a.q_len + BQ - 1) / BQ);
  const int64_t nk = (int64_t)a.batch * a.heads * ((a.kv_len + BKK - 1) / BKK);
  if (nq > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(((nq + 7) / 8) * 8)), dim3(kBThreads), C::DQ_LDS, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nk > 0)
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(((nk + 7) / 8) * 8)), dim3(kBThreads), C::DKDV_LDS, s,
                       a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_block(const BwdArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace ra
