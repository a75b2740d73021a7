// bf16 blockwise attention with online-softmax merge, gfx950 (MI355X).
//
// One workgroup owns BM = 128 query rows of one (batch, head) and streams the
// KV blocks it is given, tile by tile (BN = 64 keys), through LDS.  The state
// of the online softmax (running max m, running sum l, unnormalised output
// acc; the triple of the "Gotchas and Failure Modes" section of "Ring
// Attention: Train 1M Tokens on 8GB GPUs in 2026") lives in registers for the
// whole launch, so a fused launch over all ring blocks never round-trips it
// through HBM.
//
// Per wave (32 query rows), per tile:
//   S^T[64 keys x 32 rows] = K . Q^T      v_mfma_f32_32x32x16_bf16, K from LDS,
//                                         Q fragments held in registers
//   causal / ragged mask (diagonal and tail tiles only)
//   m' = max(m, rowmax S); p = exp2(S*c - m'); l = l*2^(m-m') + sum p;
//   acc *= 2^(m-m') (skipped when no row's max moved)      c = scale*log2(e)
//   O^T[D x 32 rows] += V^T . P^T         v_mfma_f32_32x32x16_bf16, V^T gathered
//                                         from LDS with ds_read_b64_tr_b16
// Computing S transposed puts one query row in each lane column of the MFMA
// result, so row max / row sum are per-lane scalars (plus one swap between
// the two 32-lane halves) and the S^T result registers are directly the P^T
// operand of the second product once the keys inside each 16-key step are
// permuted the same way on the V side.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;                       // 16-byte chunks per K/V row
  static constexpr int DMA_PER_WAVE = BN * D * 2 / 1024 / kWaves;  // 1 KiB LDS-DMA copies per wave per tile
  static constexpr int KS = D / 16;                      // k-steps of Q.K^T
  static constexpr int DB = D / 32;                      // 32-row blocks of O^T
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;       // K and V, double-buffered
};

// LDS placement of 16-byte chunk c of key row `key`.  K rows are read 16 bytes
// per lane, 16 rows at a time at one chunk column: XOR the column with the row
// so those 16 reads hit 16 different 16-byte bank groups.  V rows are read by
// the transpose loads 8 rows x 4 chunks at a time: XOR the 4-chunk group with
// the row so the 8 rows spread over the banks.
template <int D>
__device__ __forceinline__ int k_off(int key, int c) {
  const int cs = (D == 128) ? (c ^ (key & 15)) : (c ^ ((key >> 1) & 7));
  return key * (D * 2) + cs * 16;
}
template <int D>
__device__ __forceinline__ int v_off(int key, int c) {
  const int cs = (D == 128) ? (c ^ ((key & 3) << 2)) : (c ^ (((key >> 1) & 1) << 2));
  return key * (D * 2) + cs * 16;
}

__device__ __forceinline__ float pair_max(float x) {
  // max(x[lane], x[lane ^ 32]) on every lane
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct RowRange {
  int64_t first_pos, last_pos;  // global positions of the workgroup's first / last valid row
};

// Number of BN-key tiles of a block that some row of the workgroup can see.
__device__ __forceinline__ int block_tiles(const AttnArgs& a, int64_t pos0, const RowRange& rr) {
  int64_t nk = a.kv_len;
  if (a.causal) {
    int64_t lim = rr.last_pos - pos0 + 1;
    nk = lim < 0 ? 0 : (lim < nk ? lim : nk);
  }
  return (int)((nk + BN - 1) / BN);
}

template <int D, typename OutT, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a, BlockTable tbl) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int n_qt = (int)((a.q_len + BM - 1) / BM);
  const int n_work = a.batch * a.heads * n_qt;
  // Spread consecutive work items over one XCD: workgroups are dispatched to
  // the 8 XCDs round-robin by id, so id -> (xcd, slot) -> contiguous range per
  // XCD keeps the row tiles of one head (same K/V stream) on one L2.
  const int per = (n_work + 7) >> 3;
  const int wid = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (wid >= n_work) return;
  const int bh = wid / n_qt;
  const int qt = n_qt - 1 - (wid - bh * n_qt);  // later rows first: they see more keys
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int64_t row0 = (int64_t)qt * BM;
  const int64_t r = row0 + 32 * wave + l32;  // this lane's query row
  const bool row_ok = r < a.q_len;
  RowRange rr;
  rr.first_pos = a.q_pos0 + row0;
  rr.last_pos = a.q_pos0 + ((row0 + BM < a.q_len) ? row0 + BM : a.q_len) - 1;
  const int64_t wave_last_pos = a.q_pos0 + row0 + 32 * wave + 31;
  const int64_t my_pos = a.q_pos0 + r;
  const float c2 = a.scale * kLog2e;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds row r, d = 16ks + 8hf + 0..7
  bf16x8 qf[C::KS];
  {
    const __bf16* qp = (const __bf16*)a.q + b * a.q_sb + r * a.q_ss + h * a.q_sh + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (row_ok) {
        qf[ks] = *(const bf16x8*)(qp + 16 * ks);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[ks][j] = (__bf16)0.0f;
      }
    }
  }

  // ---- state: m2 (running max in log2 units), l (this lane's half of the sum), acc
  const int64_t sidx = ((int64_t)b * a.heads + h) * a.q_len + r;
  float m2 = -INFINITY;
  float lpart = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  // ---- tile loader: direct global -> LDS copies (global_load_lds_dwordx4).
  // One instruction moves 64 lanes x 16 bytes into 1 KiB of LDS at M0, lane i
  // filling bytes [16i, 16i+16).  Each lane therefore fetches the global chunk
  // that the swizzled layout wants in its LDS slot.  The per-lane byte offsets
  // inside a tile are loop-invariant; only keys past the end of a block (the
  // ragged last tile) are clamped onto the block's last key: their scores are
  // masked to -inf, so their values meet an exact 0 and only need to be finite.
  uint32_t dk[C::DMA_PER_WAVE], dv[C::DMA_PER_WAVE];
#pragma unroll
  for (int j = 0; j < C::DMA_PER_WAVE; ++j) {
    const int slot = (wave * C::DMA_PER_WAVE + j) * 64 + lane;
    const int key = slot / C::CH;
    const int cs = slot % C::CH;
    const int ck = k_off<D>(key, cs) / 16 - key * C::CH;  // the XOR swizzle is its own inverse
    const int cv = v_off<D>(key, cs) / 16 - key * C::CH;
    dk[j] = (uint32_t)(key * a.kv_ss * 2 + ck * 16);
    dv[j] = (uint32_t)(key * a.kv_ss * 2 + cv * 16);
  }
  const int64_t kv_head_off = ((int64_t)b * a.kv_sb + (int64_t)h * a.kv_sh) * 2;
  auto issue_tile = [&](int bi, int t, int buf) {
    const int64_t t0 = (int64_t)t * BN;
    const char* kt = (const char*)tbl.k[bi] + kv_head_off + t0 * a.kv_ss * 2;
    const char* vt = (const char*)tbl.v[bi] + kv_head_off + t0 * a.kv_ss * 2;
    char* kl = lds + buf * C::TILE_BYTES;
    char* vl = lds + (2 + buf) * C::TILE_BYTES;
    const bool ragged = t0 + BN > a.kv_len;
#pragma unroll
    for (int j = 0; j < C::DMA_PER_WAVE; ++j) {
      const int blk = wave * C::DMA_PER_WAVE + j;
      uint32_t ok = dk[j], ov = dv[j];
      if (ragged) {
        const int slot = blk * 64 + lane;
        const int key = slot / C::CH;
        const int last = (int)(a.kv_len - 1 - t0);
        const int kc = key < last ? key : last;
        const uint32_t shift = (uint32_t)((key - kc) * a.kv_ss * 2);
        ok -= shift;
        ov -= shift;
      }
      __builtin_amdgcn_global_load_lds((const void*)(kt + ok),
                                       (__attribute__((address_space(3))) void*)(kl + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vt + ov),
                                       (__attribute__((address_space(3))) void*)(vl + blk * 1024), 16, 0, 0);
    }
  };
  auto advance = [&](int& bi, int& t) -> bool {
    ++t;
    while (bi < a.nblocks && t >= block_tiles(a, tbl.pos0[bi], rr)) {
      ++bi;
      t = 0;
    }
    return bi < a.nblocks;
  };

  // ---- per-lane LDS read bases.  K: row l32 (+32 per key block, an immediate),
  // chunk 2ks+hf.  V^T via transpose loads: in each 16-lane group g, lane
  // 4t+s addresses key row t of a 4-row group and columns 4s..4s+3 of a
  // 16-column slice; it receives column (lane & 15) of those 4 rows.  Rows
  // 4*(g>>1) + t (+8 for the second load, +16 per key step, +32 per key
  // block: immediates), columns 32db + 16*(g&1) + 4s.
  int kbase[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) kbase[ks] = k_off<D>(l32, 2 * ks + hf);
  int vbase[C::DB];
  {
    const int grp = lane >> 4;
    const int tr_t = (lane >> 2) & 3;
    const int tr_s = lane & 3;
    const int key0 = 4 * (grp >> 1) + tr_t;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      vbase[db] = v_off<D>(key0, 4 * db + 2 * (grp & 1) + (tr_s >> 1)) + (tr_s & 1) * 8;
  }
  constexpr int ROWB = D * 2;  // bytes per key row in LDS

  const int64_t wave_first_pos = a.q_pos0 + row0 + 32 * wave;
  int bi = 0, t = -1;
  bool have = advance(bi, t);
  // A per-block launch (state in HBM) whose rows see no key of the block
  // leaves the state untouched.
  if (MODE == kLoadStore && !have) return;
  if (MODE == kLoadStore || MODE == kLoadFinalize) {
    if (row_ok) {
      m2 = a.m[sidx] * kLog2e;
      lpart = hf == 0 ? a.l[sidx] : 0.f;
      const float* ap = a.acc + sidx * D + 4 * hf;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4 = *(const f32x4*)(ap + 32 * db + 8 * g);
          acc[db][4 * g + 0] = v4[0];
          acc[db][4 * g + 1] = v4[1];
          acc[db][4 * g + 2] = v4[2];
          acc[db][4 * g + 3] = v4[3];
        }
    }
  }

  if (have) issue_tile(bi, t, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int buf = 0;
  while (have) {
    int nbi = bi, nt = t;
    const bool have_next = advance(nbi, nt);
    if (have_next) issue_tile(nbi, nt, buf ^ 1);

    const int64_t t0 = (int64_t)t * BN;
    const int64_t tile_pos = tbl.pos0[bi] + t0;  // global position of the tile's key 0
    const bool wave_skip = a.causal && tile_pos > wave_last_pos;
    if (!wave_skip) {
      const char* kl = lds + buf * C::TILE_BYTES;
      const char* vl = lds + (2 + buf) * C::TILE_BYTES;
      // S^T = K Q^T
      f32x16 s[2];
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *(const bf16x8*)(kl + kbase[ks] + kb * 32 * ROWB);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
        }
      }
      // mask keys past the block end and (causal) keys after this lane's row:
      // key k of the tile is live iff k < thr.
      const bool need_mask = (t0 + BN > a.kv_len) || (a.causal && tile_pos + BN - 1 > wave_first_pos);
      if (need_mask) {
        int64_t lim = a.kv_len - t0;
        if (a.causal) {
          const int64_t lc = my_pos - tile_pos + 1;
          lim = lc < lim ? lc : lim;
        }
        const int thr = (int)(lim < 0 ? 0 : (lim > BN ? BN : lim)) - 4 * hf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + 8 * (i >> 2) + (i & 3);
            if (key >= thr) s[kb][i] = -INFINITY;
          }
      }
      // online softmax (log2 domain)
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m2, mx * c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m2 - m_use);
      m2 = m_new;
      float rs = 0.f;
      bf16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c2, -m_use));
          rs += p;
          pf[kb][i >> 3][i & 7] = (__bf16)p;
        }
      lpart = lpart * alpha + rs;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const char* vp = vl + vbase[db] + (32 * kb + 16 * tp) * ROWB;
            // (Assembled with a shuffle of two bf16x4 loads: building the
            // fragment element by element from bit-cast 16-bit integers is
            // miscompiled by this toolchain, which drops half the elements.)
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * ROWB));
            const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][tp], acc[db], 0, 0, 0);
          }
        }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf ^= 1;
    bi = nbi;
    t = nt;
    have = have_next;
  }

  // ---- epilogue
  const float lsum = pair_sum(lpart);
  if (!row_ok) return;
  if (MODE == kInitStore || MODE == kLoadStore) {
    if (hf == 0) {
      a.m[sidx] = m2 * kLn2;
      a.l[sidx] = lsum;
    }
    float* ap = a.acc + sidx * D + 4 * hf;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = {acc[db][4 * g + 0], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        *(f32x4*)(ap + 32 * db + 8 * g) = v4;
      }
  } else {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    if (hf == 0) a.lse[sidx] = lsum > 0.f ? m2 * kLn2 + logf(lsum) : -INFINITY;
    OutT* op = (OutT*)a.o + b * a.o_sb + r * a.o_ss + h * a.o_sh + 4 * hf;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (sizeof(OutT) == 2) {
          bf16x4 o4;
#pragma unroll
          for (int j = 0; j < 4; ++j) o4[j] = (__bf16)(acc[db][4 * g + j] * inv);
          *(bf16x4*)(op + 32 * db + 8 * g) = o4;
        } else {
          f32x4 o4;
#pragma unroll
          for (int j = 0; j < 4; ++j) o4[j] = acc[db][4 * g + j] * inv;
          *(f32x4*)(op + 32 * db + 8 * g) = o4;
        }
      }
  }
}

template <int D, typename OutT, int MODE>
hipError_t launch_t(const AttnArgs& a, const BlockTable& t, hipStream_t s) {
  using C = Cfg<D>;
  const int64_t n_qt = (a.q_len + BM - 1) / BM;
  const int64_t n_work = (int64_t)a.batch * a.heads * n_qt;
  if (n_work == 0) return hipSuccess;
  const int64_t per = (n_work + 7) / 8;
  auto kern = attn_bf16_kernel<D, OutT, MODE>;
  static bool attr_done = false;  // set once per instantiation; the attribute is idempotent
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(per * 8)), dim3(kThreads), C::LDS_BYTES, s, a, t);
  return hipGetLastError();
}

template <int D, typename OutT>
hipError_t launch_mode(const AttnArgs& a, const BlockTable& t, int mode, hipStream_t s) {
  switch (mode) {
    case kInitFinalize: return launch_t<D, OutT, kInitFinalize>(a, t, s);
    case kInitStore: return launch_t<D, OutT, kInitStore>(a, t, s);
    case kLoadStore: return launch_t<D, OutT, kLoadStore>(a, t, s);
    default: return launch_t<D, OutT, kLoadFinalize>(a, t, s);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const BlockTable& t, int mode, hipStream_t s) {
  const bool d128 = a.head_dim == 128;
  if (a.out_bf16) return d128 ? launch_mode<128, __bf16>(a, t, mode, s) : launch_mode<64, __bf16>(a, t, mode, s);
  return d128 ? launch_mode<128, float>(a, t, mode, s) : launch_mode<64, float>(a, t, mode, s);
}

}  // namespace ra
