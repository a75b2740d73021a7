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
// Two kernels per block, eight waves per workgroup (two per SIMD, so one
// wave's MFMAs overlap another's exponentials, LDS reads and barrier), each
// streaming query or key tiles through a three-stage LDS ring of direct
// global->LDS copies:
//   dq kernel:   a workgroup owns 256 query rows (32 per wave) and streams
//                the block's 64-key tiles (tile t+2 in flight while tile t
//                is computed): S^T = K Q^T, dP^T = V dO^T, then
//                dQ^T += K^T dS^T.  Q and dO fragments stay in registers.
//   dkdv kernel: a workgroup owns 128 keys, 32 per pair of waves on one
//                SIMD, and streams 64-row query tiles with their LSE and
//                delta (tile t+1 in flight).  One wave of the pair holds K
//                fragments, forms S = Q K^T and P for tile t, accumulates
//                dV^T += dO^T P and hands P over through LDS; the other holds
//                V fragments and, one tile behind, forms dP = dO V^T,
//                dS = P (dP - delta) and accumulates dK^T += Q^T dS.  S and
//                dP are formed here and again in the dq kernel: 14 D flops
//                per visible pair against the 10 D of the five products.
// Matrix products use v_mfma_f32_32x32x16_bf16 with the same operand layouts
// as the forward kernel: transposed-operand fragments (K^T, dO^T, Q^T) come
// from LDS with ds_read_b64_tr_b16 in the 4-row-group key order that matches
// the accumulator layout of the score fragments.
#include "attn_common.h"
#include "ra_internal.h"

// The two kernels can be built as separate objects (RA_BWD_PART 1: dq, 2:
// dK/dV) so that each gets its own scheduling flags; 0 builds both.
#ifndef RA_BWD_PART
#define RA_BWD_PART 0
#endif

namespace ra {
namespace {

constexpr int kBWaves = 8;                 // waves per workgroup of the dq kernel
constexpr int kBThreads = 64 * kBWaves;
constexpr int BQ = 32 * kBWaves;           // dq kernel: query rows per workgroup
constexpr int BKN = 64;                    // dq kernel: keys per tile
constexpr int kStages = 3;                 // LDS ring depth of the dq kernel

template <int D>
struct BCfg {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int KT = BKN * ROWB;        // bytes of a 64-key tile
  // dq stage: K (u_off placement: row reads for S, transpose reads for dQ),
  // V rows (row-read placement)
  static constexpr int DQ_STAGE = 2 * KT;
  static constexpr int DQ_LDS = kStages * DQ_STAGE;
  static constexpr int DQ_CPW = DQ_STAGE / 1024 / kBWaves;  // 1 KiB copies per wave per tile
  static_assert(DQ_STAGE % (1024 * kBWaves) == 0, "copies per wave");
  static_assert(DQ_LDS <= 160 * 1024, "LDS budget");
};

// Row of element i of a 32x32 MFMA result held by a lane in half hf.
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + (i & 3) + 4 * hf; }

__device__ __forceinline__ bf16x8 pack8(const bf16x2 (&x)[16], int q0) {
  const bf16x4 lo = __builtin_shufflevector(x[q0], x[q0 + 1], 0, 1, 2, 3);
  const bf16x4 hi = __builtin_shufflevector(x[q0 + 2], x[q0 + 3], 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 pack8(const bf16x2 (&x)[8], int q0) {
  const bf16x4 lo = __builtin_shufflevector(x[q0], x[q0 + 1], 0, 1, 2, 3);
  const bf16x4 hi = __builtin_shufflevector(x[q0 + 2], x[q0 + 3], 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Clamp a 64-bit tile-relative bound into [lo, hi] as int.
__device__ __forceinline__ int clamp_i(int64_t x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : (int)x); }

#if RA_BWD_PART != 2
// ---------------------------------------------------------------------------
// dQ: one workgroup per BQ query rows of one (b, h); this lane's row r.
template <int D>
__global__ __launch_bounds__(kBThreads) void bwd_dq_kernel(BwdArgs a) {
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
  const float dlt_r = a.delta[sidx];
  wait_vm<0>();  // the register loads above, before any copy is in flight
  const bool row_live = row_ok && lse_r > -INFINITY;  // a row that saw no key anywhere has no gradient
  const float lse2 = row_live ? lse_r * kLog2e : 0.f;
  const float dlt = row_live ? dlt_r : 0.f;
  const float c2 = a.scale * kLog2e;
  // keys visible to this row: [0, klim) of the block
  int64_t klim = a.kv_len;
  if (a.causal) {
    const int64_t e = a.q_pos0 + r - a.kv_pos0 + 1;
    klim = e < klim ? e : klim;
  }
  if (!row_live) klim = 0;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  const uint32_t base = lds_addr_of(lds);
  const int64_t row_bytes = a.kv_ss * 2;
  const char* ksrc = (const char*)a.k + (b * a.kv_sb + h * a.kv_sh) * 2;
  const char* vsrc = (const char*)a.v + (b * a.kv_sb + h * a.kv_sh) * 2;
  // Copies: wave w takes the stage's 1 KiB chunks CPW w .. CPW w + CPW - 1
  // (K tile, then V tile): one contiguous run, one M0.  Per-lane global
  // offsets do not depend on the tile; the instruction offset is taken out.
  static_assert(C::DQ_CPW == 4 || C::DQ_CPW == 2, "copies per wave");
  constexpr int CPT = C::KT / 1024;  // chunks per tile
  const int w_tile = (C::DQ_CPW * wave) / CPT;  // 0: K, 1: V
  const char* w_src = w_tile == 0 ? ksrc : vsrc;
  const uint32_t w_run = (uint32_t)(C::DQ_CPW * wave) * 1024;
  uint32_t w_off[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < C::DQ_CPW; ++j) {
    const int p = ((C::DQ_CPW * wave) % CPT + j) * 1024 + lane * 16;
    const int rw = p / (D * 2);
    const int pc = (p % (D * 2)) / 16;
    const int lc = pc ^ (w_tile == 0 ? u_swz<D>(rw) : (k_off<D>(rw, pc) / 16 - rw * (D / 8)) ^ pc);
    w_off[j] = (uint32_t)(rw * row_bytes + lc * 16) - 1024u * j;  // >= 0: chunk j's rows start at >= 1 KiB j
  }
  auto issue = [&](int t, uint32_t st) {
    const int64_t go = (int64_t)t * BKN * row_bytes;
    const int valid = (int)(a.kv_len - (int64_t)t * BKN);
    if (valid >= BKN) {
      if constexpr (C::DQ_CPW == 4)
        lds_dma_x4(w_src + go, w_off, st + w_run);
      else
        lds_dma_x2(w_src + go, w_off, st + w_run);
      return;
    }
    // last, partial tile: keys past the block end re-read its last key
#pragma unroll
    for (int j = 0; j < C::DQ_CPW; ++j) {
      const int p = ((C::DQ_CPW * wave) % CPT + j) * 1024 + lane * 16;
      const int rw = p / (D * 2);
      const int pc = (p % (D * 2)) / 16;
      const int lc = pc ^ (w_tile == 0 ? u_swz<D>(rw) : (k_off<D>(rw, pc) / 16 - rw * (D / 8)) ^ pc);
      const int rr = rw < valid ? rw : valid - 1;
      lds_dma16(w_src + go, (uint32_t)(rr * row_bytes + lc * 16), st + w_run + j * 1024);
    }
  };
  // per-lane LDS offsets: K rows (u_off) and V rows (k_off) for the row
  // reads, row l32 (+32 an immediate), chunk 2 ks + hf; K^T transpose reads,
  // rows key0 (lo) and key0 + 8 (hi) of each 16-row step, column block db by
  // XOR with 64 db
  int kro[C::KS], vro[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    kro[ks] = u_off<D>(l32, 2 * ks + hf);
    vro[ks] = C::KT + k_off<D>(l32, 2 * ks + hf);
  }
  int tr_lo, tr_hi;
  {
    const int g4 = lane >> 4, tt = (lane >> 2) & 3, ss = lane & 3;
    const int key0 = 4 * (g4 >> 1) + tt;
    const int c0 = 2 * (g4 & 1) + (ss >> 1);
    tr_lo = u_off<D>(key0, c0) + (ss & 1) * 8;
    tr_hi = u_off<D>(key0 + 8, c0) + (ss & 1) * 8;
  }

  // stages rotate: tile t, t+1 (landed), t+2 (in flight)
  uint32_t st_c = base, st_1 = base + C::DQ_STAGE, st_2 = base + 2 * C::DQ_STAGE;
  issue(0, st_c);
  if (n_tiles > 1) {
    issue(1, st_1);
    wait_vm<C::DQ_CPW>();
  } else {
    wait_vm<0>();
  }
  wg_barrier();
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 2 < n_tiles) issue(t + 2, st_2);
    const int kv_rel = clamp_i(klim - (int64_t)t * BKN, 0, BKN);  // visible keys of this tile: [0, kv_rel)
    const bool full = __all(kv_rel == BKN);  // wave-uniform
    bf16x2 dsp[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for keys 32 kb .. 32 kb + 31 of the tile
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(lds_bf16x8*)(size_t)(st_c + kro[ks] + kb * 32 * (D * 2)),
                                                    qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(lds_bf16x8*)(size_t)(st_c + vro[ks] + kb * 32 * (D * 2)),
                                                     df[ks], dp, 0, 0, 0);
      }
      // dS^T = P^T (dP^T - delta), P^T = exp2(S^T c - LSE2), bf16 pairs;
      // no per-key test where every row of the wave sees the whole tile
      if (full) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float v2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int i = 2 * q + u;
            v2[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -lse2)) * (dp[i] - dlt);
          }
          dsp[8 * kb + q] = bf16x2{(__bf16)v2[0], (__bf16)v2[1]};
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float v2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int i = 2 * q + u;
            const bool vis = 32 * kb + acc_row(i, hf) < kv_rel;
            const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -lse2)) : 0.f;
            v2[u] = p * (dp[i] - dlt);
          }
          dsp[8 * kb + q] = bf16x2{(__bf16)v2[0], (__bf16)v2[1]};
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each half's operands short-lived (register budget)
    }
    // dQ^T += K^T dS^T, K^T from the same K tile by transpose reads
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const bf16x8 pf = pack8(dsp, 8 * kb + 4 * tp);
        const int row = 32 * kb + 16 * tp;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(size_t)(st_c + ((uint32_t)tr_lo ^ (64u * db)) + row * (D * 2)));
          const bf16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(size_t)(st_c + ((uint32_t)tr_hi ^ (64u * db)) + row * (D * 2)));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                            pf, acc[db], 0, 0, 0);
        }
      }
    if (t + 2 < n_tiles)
      wait_vm<C::DQ_CPW>();  // tile t+1 landed; t+2 may still be in flight
    else
      wait_vm<0>();
    wg_barrier();
    const uint32_t st_free = st_c;  // tile t's stage takes tile t+3
    st_c = st_1;
    st_1 = st_2;
    st_2 = st_free;
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

#endif  // RA_BWD_PART != 2

// ---------------------------------------------------------------------------
// dK and dV in one pass, split over wave pairs: a workgroup owns 128 keys;
// wave w (0-3, the P side) and wave w+4 (the dS side) share a SIMD and the
// same 32 keys.  For query tile t (64 rows) the P side forms S = Q K^T and P
// (from the forward's LSE), stores P as bf16 in LDS and accumulates
// dV^T += dO^T P; one trip later the dS side forms dP = dO V^T, reads that P
// (the value dV used), forms dS = P (dP - delta) and accumulates
// dK^T += Q^T dS.  Both sides hold the same key in the same lane and the
// scores in the same accumulator layout, so the hand-over is a plain per-lane
// copy.  Each stage holds the tile's Q and dO rows once, in the placement
// both read kinds take without bank conflicts (u_off): row reads for S and
// dP, transpose reads for dO^T and Q^T.  Three stages (tile t for the P side,
// t-1 for the dS side, t+1 landing) and two P buffers that alternate between
// trips.  Every wave copies one contiguous run of 1 KiB chunks per stage
// under one M0 value; the first wave of each half also copies the tile's LSE
// (P side) or delta (dS side) under the same M0, in the 256 bytes in front of
// its run.
constexpr int BQK = 64;      // dK/dV kernel: query rows per tile
constexpr int kKvStages = 3;
constexpr int BKP = 128;     // keys per workgroup (32 per wave pair)

template <int D>
struct KvStage {
  static constexpr int ROWB = 2 * D;
  static constexpr int TB = BQK * ROWB;       // bytes of a 64-row tile of Q or dO
  // LSE[64], Q tile, delta[64], dO tile
  static constexpr int LSE_OFF = 0;
  static constexpr int Q_OFF = 256;
  static constexpr int DLT_OFF = 256 + TB;
  static constexpr int DO_OFF = 512 + TB;
  static constexpr int BYTES = 512 + 2 * TB;
  static constexpr int PX_OFF = kKvStages * BYTES;
  static constexpr int PX_PAIR = BQK * 32 * 2;  // bf16 P of one pair: 64 rows x 32 keys
  static constexpr int PX_BYTES = 4 * PX_PAIR;
  static constexpr int LDS = PX_OFF + 2 * PX_BYTES;
  static constexpr int CPT = TB / 1024;          // 1 KiB chunks per tile
  static constexpr int CPW = 2 * CPT / kBWaves;  // per wave per stage: 4 (D = 128) or 2 (D = 64)
  static_assert(CPW == 4 || CPW == 2, "copies per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

#if RA_BWD_PART != 1
template <int D>
__global__ __launch_bounds__(kBThreads) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BCfg<D>;
  using S = KvStage<D>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int n_kt = (int)((a.kv_len + BKP - 1) / BKP);
  const int n_work = a.batch * a.heads * n_kt;
  const int per = (n_work + 7) >> 3;
  const int wid = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (wid >= n_work) return;
  const int bh = wid / n_kt;
  const int kt = wid - bh * n_kt;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int role = wave >> 2;  // 0: S, P, dV; 1: dP, dS, dK
  const int pair = wave & 3;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int64_t k0 = (int64_t)kt * BKP;
  const int64_t c = k0 + 32 * pair + l32;
  const bool key_ok = c < a.kv_len;
  int64_t r_min = 0;
  if (a.causal) {
    r_min = a.kv_pos0 + k0 - a.q_pos0;
    if (r_min < 0) r_min = 0;
    if (r_min >= a.q_len) return;
  }
  const int n_qt = (int)((a.q_len + BQK - 1) / BQK);
  const int qt0 = (int)(r_min / BQK);

  // K fragments (role 0) or V fragments (role 1) of this lane's key
  bf16x8 fr[C::KS];
  {
    const __bf16* src = (const __bf16*)(role == 0 ? a.k : a.v) + b * a.kv_sb + c * a.kv_ss + h * a.kv_sh + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (key_ok) {
        fr[ks] = *(const bf16x8*)(src + 16 * ks);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) fr[ks][j] = (__bf16)0.0f;
      }
    }
  }
  wait_vm<0>();  // the register loads above, before any copy is in flight
  const float c2 = a.scale * kLog2e;
  const int64_t first_row = a.causal ? a.kv_pos0 + c - a.q_pos0 : 0;  // rows >= first_row see key c
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  const uint32_t base = lds_addr_of(lds);
  const int64_t qrow_bytes = a.q_ss * 2;
  const char* qsrc = (const char*)a.q + (b * a.q_sb + h * a.q_sh) * 2;
  const char* osrc = (const char*)a.dout + (b * a.q_sb + h * a.q_sh) * 2;
  const char* lse_bh = (const char*)(a.lse + ((int64_t)b * a.heads + h) * a.q_len);
  const char* dl_bh = (const char*)(a.delta + ((int64_t)b * a.heads + h) * a.q_len);
  auto stage = [&](int t) -> uint32_t { return base + ((uint32_t)t % kKvStages) * S::BYTES; };

  // ---- copies: wave w takes chunks CPW w .. CPW w + CPW - 1 of the stage's
  // 2 CPT chunks (Q tile, then dO tile): a contiguous run, one M0.  Per-lane
  // global offsets do not depend on the tile; each has its instruction offset
  // taken out.  Waves 0 and 4 (first of the Q and dO runs) also copy LSE and
  // delta (64 rows, 4 bytes per lane) into the 256 bytes in front of the run.
  const int w_tile = (S::CPW * wave) / S::CPT;  // 0: Q, 1: dO
  const char* w_src = w_tile == 0 ? qsrc : osrc;
  const bool w_lead = (S::CPW * wave) % S::CPT == 0;  // waves 0 and 4
  const char* w_dsrc = w_tile == 0 ? lse_bh : dl_bh;
  const uint32_t w_run = (w_tile == 0 ? S::Q_OFF : S::DO_OFF) + ((S::CPW * wave) % S::CPT) * 1024;
  uint32_t w_off[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < S::CPW; ++j) {
    const int p = ((S::CPW * wave) % S::CPT + j) * 1024 + lane * 16;
    const int rw = p / S::ROWB;
    const int pc = (p % S::ROWB) / 16;
    const int lc = pc ^ u_swz<D>(rw);  // the logical chunk that the placement puts here
    // (>= 0: chunk j's rows start at or after byte 1 KiB j of the source, a
    // row being >= 128 bytes; the lead waves' extra 256 goes on the base)
    w_off[j] = (uint32_t)(rw * qrow_bytes + lc * 16) - 1024u * j;
  }
  auto issue = [&](int t, uint32_t st) {
    const int64_t row0 = (int64_t)t * BQK;
    const int64_t go = row0 * qrow_bytes;
    const int valid = (int)(a.q_len - row0);
    if (valid >= BQK) {
      if (w_lead) {  // the runs' instruction offsets are 256 + 1 KiB j: the global base moves 256 down
        if constexpr (S::CPW == 4)
          lds_dma_1x4(w_dsrc + row0 * 4, (uint32_t)lane * 4, w_src + go - 256, w_off, st + w_run - 256);
        else
          lds_dma_1x2(w_dsrc + row0 * 4, (uint32_t)lane * 4, w_src + go - 256, w_off, st + w_run - 256);
      } else {
        if constexpr (S::CPW == 4)
          lds_dma_x4(w_src + go, w_off, st + w_run);
        else
          lds_dma_x2(w_src + go, w_off, st + w_run);
      }
      return;
    }
    // last, partial tile: rows past the chunk's end re-read its last row
    if (w_lead) {
      const int rr = lane < valid ? lane : valid - 1;
      lds_dma4(w_dsrc + row0 * 4, (uint32_t)rr * 4, st + w_run - 256);
    }
#pragma unroll
    for (int j = 0; j < S::CPW; ++j) {
      const int p = ((S::CPW * wave) % S::CPT + j) * 1024 + lane * 16;
      const int rw = p / S::ROWB;
      const int pc = (p % S::ROWB) / 16;
      const int lc = pc ^ u_swz<D>(rw);
      const int rr = rw < valid ? rw : valid - 1;
      lds_dma16(w_src + go, (uint32_t)(rr * qrow_bytes + lc * 16), st + w_run + j * 1024);
    }
  };

  // ---- per-lane LDS offsets.  Row reads (S = Q K^T, dP = dO V^T): row l32
  // (+32: an immediate, u depends on the row mod 16), chunk 2 ks + hf.
  // Transpose reads (dO^T, Q^T): rows key0 (lo) and key0 + 8 (hi) of each
  // 16-row step (steps are immediates), column block db by XOR with 64 db.
  int rofs[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) rofs[ks] = u_off<D>(l32, 2 * ks + hf);
  int tr_lo, tr_hi;
  {
    const int g4 = lane >> 4, tt = (lane >> 2) & 3, ss = lane & 3;
    const int key0 = 4 * (g4 >> 1) + tt;
    const int c0 = 2 * (g4 & 1) + (ss >> 1);
    tr_lo = u_off<D>(key0, c0) + (ss & 1) * 8;
    tr_hi = u_off<D>(key0 + 8, c0) + (ss & 1) * 8;
  }
  // P hand-over: this lane's 64 bytes as four 16-byte pieces, piece j at
  // 1 KiB j + 16 lane (consecutive lanes on consecutive banks)
  const uint32_t px_lane = base + S::PX_OFF + pair * S::PX_PAIR + lane * 16;
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_w;
  typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;

  // Stage addresses rotate by trip: the P side's tile t, the dS side's t-1
  // and the copy target t+1 (which reuses t-2's stage).
  uint32_t st_p = stage(qt0), st_n = stage(qt0 + 1), st_d = stage(qt0 + 2);
  issue(qt0, st_p);
  wait_vm<0>();
  wg_barrier();
  const int n_iter = n_qt - qt0 + 1;  // the last trip serves only the dS side
  for (int i = 0; i < n_iter; ++i) {
    const int t = qt0 + i;
    if (t + 1 < n_qt) issue(t + 1, st_n);
    const int tw = role == 0 ? t : t - 1;  // this wave's tile
    if (tw >= qt0 && tw < n_qt) {
      const uint32_t st = role == 0 ? st_p : st_d;
      const int64_t row_t0 = (int64_t)tw * BQK;
      const int lo = key_ok ? clamp_i(first_row - row_t0, 0, BQK) : BQK;  // rows [lo, hi) of the tile see the key
      const int hi = clamp_i(a.q_len - row_t0, 0, BQK);
      // S = Q K^T (role 0) or dP = dO V^T (role 1), rows 0-31 and 32-63;
      // per-lane bases once per tile, rows 32-63 an immediate
      f32x16 r0 = f32x16{}, r1 = f32x16{};
      const uint32_t rows = st + (role == 0 ? S::Q_OFF : S::DO_OFF);
      uint32_t rb[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) rb[ks] = rows + rofs[ks];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        r0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(lds_bf16x8*)(size_t)rb[ks], fr[ks], r0, 0, 0, 0);
        r1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(lds_bf16x8*)(size_t)(rb[ks] + 32 * S::ROWB), fr[ks], r1, 0, 0,
                                                     0);
      }
      bf16x2 x[16];  // P (role 0) or dS (role 1) as bf16 pairs: rows of r0, then of r1
      if (role == 0) {
        // P = exp2(S c - LSE2[row]), masked.  Where every row of the tile
        // sees every key of the wave (wave-uniform), no position test is
        // needed, and exp2(-|x|) covers rows without a visible key: x =
        // S c - LSE2 <= 0 for a row's visible keys (LSE is at least each
        // visible score), while LSE = -inf makes x = +inf and P = 0.
        // (the branch is taken once for the whole tile, so that the common
        // path is one straight block the scheduler can interleave)
        const bool full = hi == BQK && __all(lo == 0);
        if (full) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x16& r = h2 == 0 ? r0 : r1;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 l4 = *(lds_f32x4*)(size_t)(st + S::LSE_OFF + (32 * h2 + 8 * g + 4 * hf) * 4);
              float v[4];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                v[j] = __builtin_amdgcn_exp2f(-__builtin_fabsf(__builtin_fmaf(r[4 * g + j], c2, -l4[j] * kLog2e)));
              x[8 * h2 + 2 * g] = bf16x2{(__bf16)v[0], (__bf16)v[1]};
              x[8 * h2 + 2 * g + 1] = bf16x2{(__bf16)v[2], (__bf16)v[3]};
            }
          }
        } else {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x16& r = h2 == 0 ? r0 : r1;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 l4 = *(lds_f32x4*)(size_t)(st + S::LSE_OFF + (32 * h2 + 8 * g + 4 * hf) * 4);
              float v[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int row = 32 * h2 + acc_row(4 * g + j, hf);
                const bool vis = row >= lo && row < hi && l4[j] > -INFINITY;
                v[j] = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(r[4 * g + j], c2, -l4[j] * kLog2e)) : 0.f;
              }
              x[8 * h2 + 2 * g] = bf16x2{(__bf16)v[0], (__bf16)v[1]};
              x[8 * h2 + 2 * g + 1] = bf16x2{(__bf16)v[2], (__bf16)v[3]};
            }
          }
        }
        const uint32_t px = px_lane + (i & 1) * S::PX_BYTES;
#pragma unroll
        for (int j = 0; j < 4; ++j) *(lds_bf16x8_w*)(size_t)(px + 1024 * j) = pack8(x, 4 * j);
      } else {
        // dS = P (dP - delta[row]), P written by the pair's other wave last trip
        const uint32_t px = px_lane + ((i - 1) & 1) * S::PX_BYTES;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // (read as bf16 elements: extracting bf16 pairs from bit-cast
          // 32-bit words is miscompiled by this toolchain, which keeps one
          // word of four)
          const bf16x8 w = *(lds_bf16x8*)(size_t)(px + 1024 * j);
          const int h2 = j >> 1, g0 = 2 * (j & 1);
          const f32x16& r = h2 == 0 ? r0 : r1;
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const int g = g0 + gg;
            const f32x4 d4 = *(lds_f32x4*)(size_t)(st + S::DLT_OFF + (32 * h2 + 8 * g + 4 * hf) * 4);
            const float pv[4] = {(float)w[4 * gg], (float)w[4 * gg + 1], (float)w[4 * gg + 2], (float)w[4 * gg + 3]};
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = pv[q] * (r[4 * g + q] - d4[q]);
            x[8 * h2 + 2 * g] = bf16x2{(__bf16)v[0], (__bf16)v[1]};
            x[8 * h2 + 2 * g + 1] = bf16x2{(__bf16)v[2], (__bf16)v[3]};
          }
        }
      }
      // dV^T += dO^T P (role 0) or dK^T += Q^T dS (role 1): four 16-row
      // steps; per-lane bases once per tile, the steps immediates
      const uint32_t trl = st + (role == 0 ? S::DO_OFF : S::Q_OFF);
      uint32_t tb_lo[C::DB], tb_hi[C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        tb_lo[db] = trl + ((uint32_t)tr_lo ^ (64u * db));
        tb_hi[db] = trl + ((uint32_t)tr_hi ^ (64u * db));
      }
#pragma unroll
      for (int tp = 0; tp < 4; ++tp) {
        const bf16x8 xf = pack8(x, 4 * tp);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x4 vlo =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(tb_lo[db] + 16 * tp * S::ROWB));
          const bf16x4 vhi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(tb_hi[db] + 16 * tp * S::ROWB));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                            xf, acc[db], 0, 0, 0);
        }
      }
    }
    wait_vm<0>();  // tile t+1 landed
    wait_lds();    // the P just written, before the other wave of the pair reads it
    wg_barrier();
    const uint32_t st_free = st_d;  // tile t-1's stage takes tile t+2
    st_d = st_p;
    st_p = st_n;
    st_n = st_free;
  }
  if (!key_ok) return;
  float* out = (role == 0 ? a.dv : a.dk) + (((int64_t)b * a.kv_cap + c) * a.heads + h) * D + 4 * hf;
  const float f = role == 0 ? 1.f : a.scale;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v4 = *(f32x4*)(out + 32 * db + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] += f * acc[db][4 * g + j];
      *(f32x4*)(out + 32 * db + 8 * g) = v4;
    }
}

#endif  // RA_BWD_PART != 1

#if RA_BWD_PART != 2
template <int D>
hipError_t launch_dq(const BwdArgs& a, hipStream_t s) {
  using C = BCfg<D>;
  static bool attr_done = false;  // set once per instantiation; the attribute is idempotent
  if (!attr_done) {
    hipError_t e =
        hipFuncSetAttribute((const void*)bwd_dq_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, C::DQ_LDS);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t nq = (int64_t)a.batch * a.heads * ((a.q_len + BQ - 1) / BQ);
  if (nq > 0)
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(((nq + 7) / 8) * 8)), dim3(kBThreads), C::DQ_LDS, s, a);
  return hipGetLastError();
}
#endif

#if RA_BWD_PART != 1
template <int D>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t s) {
  static bool attr_done = false;  // set once per instantiation; the attribute is idempotent
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       KvStage<D>::LDS);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t nk = (int64_t)a.batch * a.heads * ((a.kv_len + BKP - 1) / BKP);
  if (nk > 0)
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(((nk + 7) / 8) * 8)), dim3(kBThreads), KvStage<D>::LDS,
                       s, a);
  return hipGetLastError();
}
#endif

}  // namespace

#if RA_BWD_PART != 2
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_dq<128>(a, s) : launch_dq<64>(a, s);
}
#endif

#if RA_BWD_PART != 1
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_dkdv<128>(a, s) : launch_dkdv<64>(a, s);
}
#endif

#if RA_BWD_PART != 2
hipError_t launch_bwd_block(const BwdArgs& a, hipStream_t s) {
  hipError_t e = launch_bwd_dq(a, s);
  return e != hipSuccess ? e : launch_bwd_dkdv(a, s);
}
#endif

}  // namespace ra
