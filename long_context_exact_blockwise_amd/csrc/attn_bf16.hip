// bf16 blockwise attention with online-softmax merge, gfx950 (MI355X).
//
// One workgroup (8 waves) owns BM = 256 query rows of one (batch, head) and
// streams the KV blocks it is given, tile by tile (BN = 64 keys), through LDS.
// The state of the online softmax (reference m, running sum l, unnormalised
// output acc; the triple of the "Gotchas and Failure Modes" section of "Ring
// Attention: Train 1M Tokens on 8GB GPUs in 2026") lives in registers for the
// whole launch, so a fused launch over all ring blocks never round-trips it
// through HBM.
//
// Per wave (32 query rows), per tile:
//   S^T[64 keys x 32 rows] = K . Q^T      v_mfma_f32_32x32x16_bf16, K from LDS,
//                                         Q fragments held in registers
//   causal / ragged mask (diagonal and tail tiles only)
//   p = exp2(S*c - m); l += sum p (fp32)  c = scale*log2(e), m a reference
//                                         point (see softmax_redo)
//   O^T[D x 32 rows] += V^T . P^T         v_mfma_f32_32x32x16_bf16, V^T gathered
//                                         from LDS with ds_read_b64_tr_b16
// Computing S transposed puts one query row in each lane column of the MFMA
// result, so row sums are per-lane scalars (plus one swap between the two
// 32-lane halves) and the S^T result registers are directly the P^T operand
// of the second product once the keys inside each 16-key step are permuted
// the same way on the V side.
//
// Software pipeline: a wave's work on tile t is a chain (S_t, softmax of S_t,
// P_t V_t), so run in order the matrix cores idle during the softmax.  Block t
// of the main loop instead issues three independent pieces of work, which the
// scheduler interleaves instruction by instruction:
//   O^T += V_{t-1}^T P_{t-1}^T   (P from the previous block)
//   S_{t+1}^T = K_{t+1} Q^T
//   softmax of S_t -> P_t        (vector ALU: exp2, bf16 pack, row sums)
#include <type_traits>

#include "attn_common.h"
#include "ra_internal.h"

namespace ra {
namespace {


constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 32 * kWaves;  // query rows per workgroup
constexpr int BN = 64;           // keys per tile

// K/V slots in LDS: slot s = (K_s, V_{s-2}) lives in buffer s % kBufs and is
// read in block s-1.  Block t copies slot t + kBufs into the buffer of slot t
// (read in block t-1) and waits for slot t+2 before the barrier that ends it,
// so kBufs-2 slots stay in flight across barriers.  Slots past the last tile
// (and the V part of slots 0, 1) copy a real tile whose products are
// discarded or multiplied by P = 0: every block issues the same number of
// copies and the wait counts stay exact.
// (Four slots, 128 KiB at D = 128; three and five measured 1.4% and 1.2%
// slower.)
#ifndef RA_SP_BUFS
#define RA_SP_BUFS 4
#endif
constexpr int kBufs = RA_SP_BUFS;

template <int D>
struct Cfg {
  static constexpr int CH = D / 8;   // 16-byte chunks per K/V row
  static constexpr int KS = D / 16;  // k-steps of Q.K^T
  static constexpr int DB = D / 32;  // 32-row blocks of O^T
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int SLOT_BYTES = 2 * TILE_BYTES;
  static constexpr int LDS_BYTES = kBufs * SLOT_BYTES;
  static constexpr int DPW = TILE_BYTES / 1024 / kWaves;  // 1 KiB copies per wave per K (or V) tile
  // In a slot, wave w's K chunks w*DPW + j and V chunks w*DPW + j sit
  // together (K first) in a 2*DPW KiB region: byte lin of the row-major
  // (swizzled) K or V tile maps to these slot offsets.  A linear offset that
  // is a multiple of DPW KiB maps to twice itself.
  static __device__ __forceinline__ int k_at(int lin) {
    const int blk = lin >> 10;
    return (blk / DPW) * (2 * DPW * 1024) + (blk % DPW) * 1024 + (lin & 1023);
  }
  static __device__ __forceinline__ int v_at(int lin) { return k_at(lin) + DPW * 1024; }
  // Slot offset of 8 key rows further down (the second half of a V^T
  // fragment): doubled when 8 rows span a wave's DPW chunks, unchanged when
  // they stay inside one wave's region.
  static constexpr int HI8 = (8 * D * 2 / 1024 >= DPW) ? 2 * 8 * D * 2 : 8 * D * 2;
};



// Row-sum bound of one tile under a stale reference: while every p of the
// tile stays <= 2^12 the reference may lag the running max.
constexpr float kPLim = 4096.0f;

// Exponentiate the 32 raw scores q.k (two f32x16 fragments of S^T) this lane
// holds for its query row against reference mref (log2 units): bf16 pairs
// p[q] = (p_{2q}, p_{2q+1}) for the P.V product; returns the fp32 sum of the
// unrounded values (the row sum, hence LSE, keeps fp32 accuracy; O then
// differs from an exactly normalised bf16-P average by at most the bf16
// rounding of P).  The other 32 keys of the tile sit in the lane 32 away.
__device__ __forceinline__ float softmax_exp(const f32x16 (&s)[2], float c2, float mref, bf16x2 (&p)[16]) {
  float rsq[4];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = 2 * q;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 4][e & 15], c2, -mref));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 4][(e & 15) + 1], c2, -mref));
    p[q] = bf16x2{(__bf16)p0, (__bf16)p1};
    // (the four partial sums start from the first pairs, not from 0: x + 0
    // cannot be folded away, since -0 + 0 is +0)
    rsq[q & 3] = q < 4 ? p0 + p1 : rsq[q & 3] + (p0 + p1);
  }
  return (rsq[0] + rsq[1]) + (rsq[2] + rsq[3]);
}

// The state is (m2, l, acc) with m2 a reference point in log2 units: l and acc
// are sums of exp2(s*c - m2).  Any m2 gives the same acc/l and m2 + log2 l, so
// m2 is moved only when it must be: a tile is first exponentiated against the
// current m2 (softmax_exp), and only if some lane of the wave then sees a row
// sum above kPLim (the max has grown by more than 12 in log2 units, or
// overflowed), or still has no reference (m2 = -inf), does softmax_redo raise
// m2 to the running max, exponentiate the tile again and rescale acc and l.
// m2 never exceeds the running max (it is only ever set to it), so l >= 1
// once a key was seen.  Returns the tile's row sum against the final m2.
template <int DB>
__device__ __forceinline__ float softmax_redo(const f32x16 (&s)[2], float c2, float& m2, float& lpart,
                                              f32x16 (&acc)[DB], bf16x2 (&p)[16]) {
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m2, mx * c2);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m2 - m_use);
  m2 = m_new;
  lpart *= alpha;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
  return softmax_exp(s, c2, m_use, p);
}


// A wave's share of one K/V slot with a single M0 value: DPW 1 KiB chunks of
// K at m0 + 1 KiB j and DPW chunks of V at m0 + 1 KiB (DPW + j).  The
// instruction offset moves the LDS destination and the global address alike,
// so lane offsets are passed with that offset taken out (ko_j = K offset -
// 1 KiB j) and the V base is passed 1 KiB DPW low.  Changing M0 while copies
// are in flight stalls the wave, so it is set once per slot.  The loads read
// the bases from copies made by s_mov_b64 inside the block: an SGPR written
// by a VALU instruction (v_readfirstlane here, v_readlane for a spilled SGPR)
// may be read by a VMEM instruction only five wait states later, which the
// compiler does not insert inside inline assembly; one written by a scalar
// instruction needs none.
template <int DPW>
__device__ __forceinline__ void lds_dma_slot(const char* kbase, const char* vbase, const uint32_t (&ko)[DPW],
                                             const uint32_t (&vo)[DPW], uint32_t m0) {
  const char* vbase_low = vbase - DPW * 1024;  // V chunks use offsets 1 KiB (DPW + j)
  const uint64_t kb = (uint64_t)kbase, vb = (uint64_t)vbase_low;
  const uint32_t klo = __builtin_amdgcn_readfirstlane((uint32_t)kb);
  const uint32_t khi = __builtin_amdgcn_readfirstlane((uint32_t)(kb >> 32));
  const uint32_t vlo = __builtin_amdgcn_readfirstlane((uint32_t)vb);
  const uint32_t vhi = __builtin_amdgcn_readfirstlane((uint32_t)(vb >> 32));
  const uint64_t kbs = ((uint64_t)khi << 32) | klo;
  const uint64_t vbs = ((uint64_t)vhi << 32) | vlo;
  uint32_t saved;
  uint64_t tk, tv;
  if constexpr (DPW == 2) {
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[m0]\n\t"
        "s_mov_b64 %[tk], %[kb]\n\t"
        "s_mov_b64 %[tv], %[vb]\n\t"
        "global_load_lds_dwordx4 %[k0], %[tk]\n\t"
        "global_load_lds_dwordx4 %[k1], %[tk] offset:1024\n\t"
        "global_load_lds_dwordx4 %[v0], %[tv] offset:2048\n\t"
        "global_load_lds_dwordx4 %[v1], %[tv] offset:3072\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved), [tk] "=&s"(tk), [tv] "=&s"(tv)
        : [k0] "v"(ko[0]), [k1] "v"(ko[1]), [v0] "v"(vo[0]), [v1] "v"(vo[1]),
          [m0] "s"(__builtin_amdgcn_readfirstlane(m0)), [kb] "s"(kbs), [vb] "s"(vbs)
        : "memory");
  } else {
    static_assert(DPW == 1, "one or two chunks per wave");
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[m0]\n\t"
        "s_mov_b64 %[tk], %[kb]\n\t"
        "s_mov_b64 %[tv], %[vb]\n\t"
        "global_load_lds_dwordx4 %[k0], %[tk]\n\t"
        "global_load_lds_dwordx4 %[v0], %[tv] offset:1024\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved), [tk] "=&s"(tk), [tv] "=&s"(tv)
        : [k0] "v"(ko[0]), [v0] "v"(vo[0]), [m0] "s"(__builtin_amdgcn_readfirstlane(m0)), [kb] "s"(kbs),
          [vb] "s"(vbs)
        : "memory");
  }
}


struct RowRange {
  int64_t first_pos, last_pos;  // global positions of the workgroup's first / last valid row
};

// Number of BN-key tiles of a block (len valid keys from pos0) that some row of
// the workgroup can see.
__device__ __forceinline__ int block_tiles(const AttnArgs& a, int64_t pos0, int len, const RowRange& rr) {
  int64_t nk = len;
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
  constexpr int ROWB = D * 2;
  constexpr int DPW = C::DPW;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int64_t row0 = (int64_t)qt * BM;
  const int64_t r = row0 + 32 * wave + l32;  // this lane's query row
  const bool row_ok = r < a.q_len;
  RowRange rr;
  rr.first_pos = a.q_pos0 + row0;
  rr.last_pos = a.q_pos0 + ((row0 + BM < a.q_len) ? row0 + BM : a.q_len) - 1;
  const float c2s = a.scale * kLog2e;

  int n_tiles = 0;
  for (int bi = 0; bi < a.nblocks; ++bi) n_tiles += block_tiles(a, tbl.pos0[bi], tbl.len[bi], rr);
  // A per-block launch (state in HBM) whose rows see no key of the block
  // leaves the state untouched.
  if (MODE == kLoadStore && n_tiles == 0) return;

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
  // ---- state: m2 (reference, log2 units), l (this lane's half of the sum), acc
  const int64_t sidx = ((int64_t)b * a.heads + h) * a.q_len + r;
  float m2 = -INFINITY;
  float lpart = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  if ((MODE == kLoadStore || MODE == kLoadFinalize) && row_ok) {
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

  if (n_tiles > 0) {
    // ---- tile cursors (all wave-uniform, scalar): block, tile, visible tile
    // count, the block's valid keys (< 2^30, checked on the host) and its
    // ragged last tile (-1: none), position of the tile's key 0 relative to
    // the workgroup's first row (clamped below: far-away tiles are fully
    // visible) and, for the copy cursors, the global address of the tile for
    // this (b, h).
    struct Cur {
      int b, t, n, len, ragged, rel;
      const char* src;
    };
    const int64_t kv_head_off = ((int64_t)b * a.kv_sb + (int64_t)h * a.kv_sh) * 2;
    const int64_t tile_bytes_g = (int64_t)BN * a.kv_ss * 2;
    auto seek = [&](Cur& c, int which) {  // which: 0 none, 1 K, 2 V
      while (c.b < a.nblocks && (c.n = block_tiles(a, tbl.pos0[c.b], tbl.len[c.b], rr)) == 0) ++c.b;
      c.t = 0;
      if (c.b < a.nblocks) {
        c.len = tbl.len[c.b];
        c.ragged = (c.len & (BN - 1)) ? (c.len >> 6) : -1;  // the ragged tile of a block is its last one
        // visible tiles start at or before the last row; far below, clamp so
        // that rel + 64 t stays far below for every tile of the block
        const int64_t rel = tbl.pos0[c.b] - rr.first_pos;
        c.rel = rel < (int64_t)INT32_MIN + 64 ? INT32_MIN + 64 : (int)rel;
        if (which) c.src = (const char*)(which == 2 ? tbl.v[c.b] : tbl.k[c.b]) + kv_head_off;
      }
    };
    auto step = [&](Cur& c, int which) {
      if (++c.t < c.n) {
        c.rel += BN;
        c.src += tile_bytes_g;
      } else {
        ++c.b;
        seek(c, which);
      }
    };

    // ---- copies into LDS.  Copy j of a wave's K (or V) share moves 1 KiB =
    // 64 lanes x 16 bytes: LDS chunk blk = wave*DPW + j of the row-major tile,
    // lane i fetching the global chunk that the swizzled layout puts at byte
    // 16 i of it.
    // dkj / dvj: the offsets with the instruction offset 1 KiB j taken out
    // (chunk j's key rows start at >= 1 KiB j of the source, a row being >=
    // D*2 bytes, so they stay non-negative)
    uint32_t dkj[DPW], dvj[DPW];
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int slot = (wave * DPW + j) * 64 + lane;
      const int key = slot / C::CH;
      const int cs = slot % C::CH;
      dkj[j] = (uint32_t)(key * a.kv_ss * 2 + (k_off<D>(key, cs) / 16 - key * C::CH) * 16) - 1024u * j;
      dvj[j] = (uint32_t)(key * a.kv_ss * 2 + (v_off<D>(key, cs) / 16 - key * C::CH) * 16) - 1024u * j;
    }
    const uint32_t lds_base = lds_addr_of(lds);
    const uint32_t lds0 = lds_base + wave * (2 * DPW * 1024);  // this wave's region of a slot
    // Ragged tile: keys past the block end re-read its last key (masked
    // later); one chunk at a time with its own M0.
    auto copy_ragged = [&](const Cur& c, bool is_v, uint32_t dst) {
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        const int key = ((wave * DPW + j) * 64 + lane) / C::CH;
        const int last = c.len - 1 - c.t * BN;
        const uint32_t off =
            (is_v ? dvj[j] : dkj[j]) + 1024u * j - (uint32_t)((key > last ? key - last : 0) * a.kv_ss * 2);
        lds_dma16(c.src, off, dst + (is_v ? DPW + j : j) * 1024);
      }
    };
    // copy cursors: K of slot s is tile min(s, n-1); V of slot s is tile
    // clamp(s-2, 0, n-1)
    Cur ck{0, 0, 0, 0, 0, 0, nullptr}, cv{0, 0, 0, 0, 0, 0, nullptr};
    seek(ck, 1);
    seek(cv, 2);
    int kidx = 0, vidx = 0;
    // (slots are never negative: the unsigned remainder is one AND)
    auto slot_dst = [&](int s) -> uint32_t { return lds0 + ((uint32_t)s % kBufs) * C::SLOT_BYTES; };
    auto copy_slot = [&](int s) {
      const uint32_t dst = slot_dst(s);
      if (ck.t != ck.ragged && cv.t != cv.ragged) {
        lds_dma_slot<DPW>(ck.src, cv.src, dkj, dvj, dst);
      } else {
        copy_ragged(ck, false, dst);
        copy_ragged(cv, true, dst);
      }
      if (kidx < n_tiles - 1) {
        step(ck, 1);
        ++kidx;
      }
      if (s >= 2 && vidx < n_tiles - 1) {
        step(cv, 2);
        ++vidx;
      }
    };
    auto slot_at = [&](int s) -> uint32_t { return lds_base + ((uint32_t)s % kBufs) * C::SLOT_BYTES; };

    // ---- per-lane LDS byte offsets inside a slot.  K: row l32 (+32 per key
    // block), chunk 2ks+hf: kofs[ks].  V^T via transpose loads: in each
    // 16-lane group g, lane 4t+s addresses key row t of a 4-row group and
    // columns 4s..4s+3 of a 16-column slice; it receives column (lane & 15)
    // of those 4 rows.  Rows 4*(g>>1) + t (+8 for the second load, +16 per
    // key step, +32 per key block), columns 32db + 16*(g&1) + 4s: vofs[db].
    // Row offsets of 16 and 32 rows are multiples of DPW KiB, which the slot
    // layout doubles; 8 rows is C::HI8.  Each tile forms the per-lane bases
    // slot + kofs[ks] and slot + vofs[db] once; the row offsets are
    // instruction immediates on top of them.
    int kofs[C::KS], vofs[C::DB];
    {
      const int kA = k_off<D>(l32, hf);
      const int g4 = lane >> 4;
      const int tr_t = (lane >> 2) & 3;
      const int tr_s = lane & 3;
      const int key0 = 4 * (g4 >> 1) + tr_t;
      const int vA = v_off<D>(key0, 2 * (g4 & 1) + (tr_s >> 1)) + (tr_s & 1) * 8;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) kofs[ks] = C::k_at(kA ^ (32 * ks));
#pragma unroll
      for (int db = 0; db < C::DB; ++db) vofs[db] = C::v_at(vA ^ (64 * db));
    }
    // V^T fragment at per-lane base `base` (slot + vofs[db]), key rows `row`..
    // (Assembled with a shuffle of two bf16x4 loads: building the fragment
    // element by element from bit-cast 16-bit integers is miscompiled by this
    // toolchain, which drops half the elements.)
    auto v_frag = [&](uint32_t base, int row) -> bf16x8 {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(base + 2 * row * ROWB));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(base + 2 * row * ROWB + C::HI8));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16 s_cur[2], s_nxt[2];     // S^T of tile t (softmax now) and t+1 (being computed)
    bf16x2 p_prev[16], p_cur[16];  // P of tile t-1 (P.V now) and t (being produced)
#pragma unroll
    for (int q = 0; q < 16; ++q) p_prev[q] = bf16x2{(__bf16)0.0f, (__bf16)0.0f};

    auto qk_products = [&](uint32_t sl, f32x16 (&sn)[2]) {
      // per-lane bases of this slot, once per tile; the second 32 keys are
      // an instruction immediate
      uint32_t kb_base[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) kb_base[ks] = sl + kofs[ks];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *(lds_bf16x8*)(size_t)(kb_base[ks] + 2 * kb * 32 * ROWB), qf[ks], ks == 0 ? f32x16{} : sn[kb], 0, 0, 0);
    };
    auto pv_products = [&](uint32_t sl, const bf16x2 (&pp)[16]) {
      // per-lane bases of this slot, once per tile; rows are instruction
      // immediates (at most 48 rows + 8 rows of one slot, < 64 KiB)
      uint32_t vb[C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) vb[db] = sl + vofs[db];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          const int q0 = 8 * kb + 4 * tp;
          const bf16x4 p_lo = __builtin_shufflevector(pp[q0], pp[q0 + 1], 0, 1, 2, 3);
          const bf16x4 p_hi = __builtin_shufflevector(pp[q0 + 2], pp[q0 + 3], 0, 1, 2, 3);
          const bf16x8 pf = __builtin_shufflevector(p_lo, p_hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vb[db], 32 * kb + 16 * tp), pf, acc[db], 0, 0, 0);
        }
    };

    // ---- prologue: slots 0 .. kBufs-1; wait for slots 0 and 1; S_0
    for (int s = 0; s < kBufs; ++s) copy_slot(s);
    wait_vm<(kBufs - 2) * 2 * DPW>();
    wg_barrier();
    qk_products(slot_at(0), s_cur);
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();  // buffer 0 is refilled by block 0

    Cur cs{0, 0, 0, 0, 0, 0, nullptr};  // tile t (softmax, mask)
    seek(cs, 0);
    const int wrow0 = 32 * wave;    // this wave's first row, relative to the workgroup
    const int myrow = wrow0 + l32;  // this lane's row, relative to the workgroup
    // One tile: S of tile t in sc (softmax now), S of t+1 into sn, P of t-1
    // in pp (P.V now), P of t into pc.  The loop runs two tiles per trip
    // with the register sets swapping roles, so no copies rotate them.
    //
    // Fast tiles (kFast) are the tiles of a run (see fast_run): neither copy
    // cursor reaches the end of its block, a ragged tile or the last tile,
    // and the compute tile needs no mask, so the tile issues its copies
    // straight from the cursors, and its only bookkeeping is two pointer
    // increments placed before the barrier, where waves wait anyway.  The
    // tile counters of the cursors are advanced once per run.  Checked tiles
    // step every cursor with all its tests (block ends, ragged tiles, the
    // clamp at the last tile) and apply the mask where a tile needs one.
    auto tile = [&](auto fast_tag, int t, f32x16 (&sc)[2], f32x16 (&sn)[2], const bf16x2 (&pp)[16],
                    bf16x2 (&pc)[16]) {
      constexpr bool kFast = decltype(fast_tag)::value;
      if constexpr (kFast) {
        lds_dma_slot<DPW>(ck.src, cv.src, dkj, dvj, slot_dst(t + kBufs));
      } else {
        copy_slot(t + kBufs);
      }
      __builtin_amdgcn_sched_barrier(0);
      // mask keys past the block end and (causal) keys after this lane's row:
      // key k of the tile is live iff k < thr
      if (!kFast && (cs.t == cs.ragged || (a.causal && cs.rel + (BN - 1) > wrow0))) {
        int lim = cs.t == cs.ragged ? cs.len - cs.t * BN : BN;
        if (a.causal) {
          const int lc = myrow - cs.rel + 1;
          lim = lc < lim ? lc : lim;
        }
        const int thr = (lim < 0 ? 0 : lim) - 4 * hf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb + 8 * (i >> 2) + (i & 3) >= thr) sc[kb][i] = -INFINITY;
      }
      __builtin_amdgcn_sched_barrier(0);
      // interleaved: P.V of tile t-1, S of tile t+1, softmax of tile t
      const float mref = m2 == -INFINITY ? 0.f : m2;
      pv_products(slot_at(t + 1), pp);
      qk_products(slot_at(t + 1), sn);
      float rs = softmax_exp(sc, c2s, mref, pc);
      __builtin_amdgcn_iglp_opt(3);
      __builtin_amdgcn_sched_barrier(0);
      if (__any(!(rs <= kPLim) || m2 == -INFINITY)) {
        // (the packed P of the common path is consumed here so that the
        // compiler forms it inside the interleaved region above instead of
        // sinking the conversions past this rare branch, which kept 32 fp32
        // values live and put 16 conversions before the barrier)
#pragma unroll
        for (int q = 0; q < 16; ++q) asm volatile("" ::"v"(pc[q]));
        rs = softmax_redo<C::DB>(sc, c2s, m2, lpart, acc, pc);
      }
      lpart += rs;
      if constexpr (kFast) {
        ck.src += tile_bytes_g;
        cv.src += tile_bytes_g;
      }
      // slot t+2 (read by tile t+1) has landed; kBufs-2 newer slots may fly
      wait_vm<(kBufs - 2) * 2 * DPW>();
      wg_barrier();
      if constexpr (!kFast) step(cs, 0);
    };
    // Tiles from t on that can run as fast tiles: each copies the tiles
    // under the copy cursors and then steps them inside their blocks (a
    // ragged tile is always a block's last), without reaching the last tile;
    // the compute tiles stay inside their block and before the first tile
    // this wave must mask (causal: the first whose last key lies past the
    // wave's first row).
    auto fast_run = [&](int t) -> int {
      int64_t r = (int64_t)ck.n - 1 - ck.t;
      r = r < (int64_t)n_tiles - 1 - kidx ? r : (int64_t)n_tiles - 1 - kidx;
      r = r < (int64_t)cv.n - 1 - cv.t ? r : (int64_t)cv.n - 1 - cv.t;
      r = r < (int64_t)n_tiles - 1 - vidx ? r : (int64_t)n_tiles - 1 - vidx;
      r = r < (int64_t)cs.n - 1 - cs.t ? r : (int64_t)cs.n - 1 - cs.t;
      if (a.causal) {
        const int64_t room = (int64_t)wrow0 - (BN - 1) - cs.rel;  // tile j is unmasked iff rel_j + 63 <= wrow0
        const int64_t nm = room < 0 ? 0 : room / BN + 1;
        r = r < nm ? r : nm;
      }
      r = r < (int64_t)n_tiles - t ? r : (int64_t)n_tiles - t;
      return r < 0 ? 0 : (int)r;
    };
    constexpr std::true_type kFastTile{};
    constexpr std::false_type kCheckedTile{};
    int t = 0;
    while (t + 1 < n_tiles) {
      const int run = fast_run(t) & ~1;
      for (int i = 0; i < run; i += 2) {
        tile(kFastTile, t + i, s_cur, s_nxt, p_prev, p_cur);
        tile(kFastTile, t + i + 1, s_nxt, s_cur, p_cur, p_prev);
      }
      ck.t += run;
      kidx += run;
      cv.t += run;
      vidx += run;
      cs.t += run;
      cs.rel += run * BN;
      t += run;
      if (t + 1 < n_tiles) {
        tile(kCheckedTile, t, s_cur, s_nxt, p_prev, p_cur);
        tile(kCheckedTile, t + 1, s_nxt, s_cur, p_cur, p_prev);
        t += 2;
      }
    }
    if (t < n_tiles) {
      tile(kCheckedTile, t, s_cur, s_nxt, p_prev, p_cur);
#pragma unroll
      for (int q = 0; q < 16; ++q) p_prev[q] = p_cur[q];  // the last tile's P, for the final P.V
    }
    // P.V of the last tile (slot n+1 holds V_{n-1})
    pv_products(slot_at(n_tiles + 1), p_prev);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<0>();
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
  const int64_t n_qt = (a.q_len + BM - 1) / BM;
  const int64_t n_work = (int64_t)a.batch * a.heads * n_qt;
  if (n_work == 0) return hipSuccess;
  const int64_t per = (n_work + 7) / 8;
  auto kern = attn_bf16_kernel<D, OutT, MODE>;
  static bool attr_done = false;  // set once per instantiation; the attribute is idempotent
  if (!attr_done) {
    hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg<D>::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(per * 8)), dim3(kThreads), Cfg<D>::LDS_BYTES, s, a, t);
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
