// Blockwise feedforward of one device's chunk, bf16, gfx950.
//
// "Ring Attention with Blockwise Transformers for Near-Infinite Context"
// (Abstract) computes the feedforward blockwise, like the attention.  The
// network is the position-wise y = gelu(x W1^T + b1) W2^T + b2 (tanh-form
// GELU; W1 [F, d], W2 [d, F], rows are output features).  The chunk's rows
// are processed in blocks; per block the hidden activation [rows, F] lives in
// a caller workspace (bf16, as P is rounded before its product in the
// attention), so memory holds one block's activation, not the chunk's.
//
// Both layers are the same kernel: C[M, N] = A[M, K] B[N, K]^T + bias[N]
// (then GELU for the first layer), bf16 in, fp32 accumulation, bf16 out.  A
// workgroup of eight waves owns a 256 x 256 tile of C at a time; a wave owns
// 64 rows x 128 columns as 2 x 4 products of v_mfma_f32_32x32x16_bf16,
// computed transposed (C^T = B A^T) so that a lane holds one row of C and
// stores runs of 4 consecutive columns.  K advances 64 at a time through two
// LDS stages filled by direct global->LDS copies, the next stage's copy in
// flight while the current one is multiplied.  The workgroups are
// persistent (one per CU), walking their XCD's run of tiles; the first copy
// of a workgroup's next tile runs beside the epilogue of the current one.
#include "attn_common.h"
#include "ra_internal.h"

namespace ra {
namespace {

// Eight waves, two per SIMD, of 64 rows x 128 columns.  (Four waves of
// 128 x 128, one per SIMD, with half the LDS operand traffic per product,
// measured 9-19% slower in several forms: with one wave per SIMD nothing
// covers a wave's barrier, operand waits and epilogue.)
constexpr int WTN = 4;                            // 32-column products per wave (128 columns)
constexpr int WTM = 2;                            // 32-row products per wave (64 rows)
constexpr int kGWaves = (256 / (32 * WTN)) * (256 / (32 * WTM));
constexpr int kGThreads = 64 * kGWaves;
constexpr int GBM = 256;                          // rows of C per workgroup
constexpr int GBN = 256;                          // columns of C per workgroup
constexpr int GBK = 64;                           // contraction per stage
constexpr int G_TILE = 256 * GBK * 2;             // 32 KiB: one operand tile (256 rows x 128 B)
constexpr int G_STAGE = 2 * G_TILE;               // weights tile, then token tile
constexpr int G_BIAS = 2 * G_STAGE;               // two 512-byte bias slices (tile parity) after the stages
constexpr int G_LDS = G_BIAS + 2 * GBN * 2;        // 129 KiB
static_assert(G_STAGE / 1024 / kGWaves == 8, "two four-copy groups per wave and stage");
static_assert((GBK / 16) % 2 == 0, "a k-tile ends on operand buffer 1, so the next one starts on buffer 0");

// GELU, tanh form (Hendrycks and Gimpel): 0.5 x (1 + tanh(u)) with u =
// sqrt(2/pi) (x + 0.044715 x^3), evaluated as x / (1 + e^(-2u)) (the same
// function, since 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u))), with e^(-2u) =
// 2^(x (c1 + c2 x^2)); both saturations are exact (e^(-2u) -> inf gives -0,
// -> 0 gives x).
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float c1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;  // -2 log2(e) sqrt(2/pi)
  constexpr float c2 = c1 * 0.044715f;
  const float e = __builtin_amdgcn_exp2f(x * __builtin_fmaf(c2, x * x, c1));
  return x * __builtin_amdgcn_rcpf(1.f + e);
}

template <bool GELU>
__global__ __launch_bounds__(kGThreads) void gemm_bt_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tiles_n = (g.n + GBN - 1) / GBN;
  const int64_t tiles_m = (g.m + GBM - 1) / GBM;
  const int64_t n_work = tiles_m * tiles_n;
  const int64_t per = (n_work + 7) >> 3;
  // Persistent workgroups: the grid is a multiple of 8 and consecutive
  // workgroups go to different XCDs.  Each XCD takes a contiguous run of
  // tiles (row-major over groups of (m tile, n tile), below); its nslots
  // workgroups walk the run together, workgroup `slot` taking tiles slot,
  // slot + nslots, ..., so the tiles in flight on an XCD are consecutive and
  // share token and weight tiles in its L2.
  const int xcd = (int)(blockIdx.x & 7);
  const int slot = (int)(blockIdx.x >> 3);
  const int nslots = (int)(gridDim.x >> 3);
// Row tiles per group of the tile order (4 measured best; 1, 8 and 16 were
// 3%, 5% and 16% slower).
#ifndef RA_FFN_GM
#define RA_FFN_GM 4
#endif
  const int64_t gspan = (int64_t)RA_FFN_GM * tiles_n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int wn = wave & 1;   // 128-column half of the tile
  const int wm = wave >> 1;  // 64-row slice of the tile
  const uint32_t base = lds_addr_of(lds);
  const int nk = g.k / GBK;

  // tile i of this workgroup: (m tile, n tile) in groups of GM row tiles:
  // consecutive ids walk GM row tiles, then the next column tile
  auto tile_of = [&](int64_t i, int64_t& m0, int& n0) -> bool {
    const int64_t r = (int64_t)slot + i * nslots;
    const int64_t wid = (int64_t)xcd * per + r;
    if (r >= per || wid >= n_work) return false;
    const int64_t grp = wid / gspan;
    const int64_t first_m = grp * RA_FFN_GM;
    const int gsize = (int)(tiles_m - first_m < RA_FFN_GM ? tiles_m - first_m : RA_FFN_GM);
    const int64_t in_g = wid - grp * gspan;
    m0 = (first_m + in_g % gsize) * GBM;
    n0 = (int)(in_g / gsize) * GBN;
    return true;
  };

  // Copies: a stage is 64 chunks of 1 KiB (8 rows x 128 B), chunks 0-31 the
  // weight tile, 32-63 the token tile; wave w copies chunks 8w .. 8w + 7 as
  // two four-copy groups, each under one M0.  Lane i of chunk q fills LDS
  // bytes 16 i of it: row 8 q + i / 8, slot i % 8, which holds the global
  // chunk the k_off placement puts there (its XOR is self-inverse).  Rows
  // past the matrix edge re-read its last row (their products are never
  // stored).  A group's instruction offsets add 1 KiB j to both addresses,
  // so the lane offsets have 1 KiB j taken out; the source base sits 3 KiB
  // before the tile's first row so that they stay non-negative when a
  // clamped row is below 8 j (the addresses formed are the rows' own).
  const bool cp_x = wave >= 4;
  const int64_t rowb = (cp_x ? g.lda : g.ldb) * 2;
  struct Src {
    const char* p;
    uint32_t off[2][4];
  };
  auto src_of = [&](int64_t m0, int n0, Src& c) {
    c.p = (cp_x ? (const char*)(g.a + m0 * g.lda) : (const char*)(g.b + (int64_t)n0 * g.ldb)) - 3072;
    const int valid = cp_x ? (int)(g.m - m0 < GBM ? g.m - m0 : GBM) : (g.n - n0 < GBN ? g.n - n0 : GBN);
#pragma unroll
    for (int gq = 0; gq < 2; ++gq)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = 8 * (wave & 3) + 4 * gq + j;
        const int row = 8 * q + (lane >> 3);
        const int col = k_off<64>(row, lane & 7) / 16 - row * 8;
        const int rr = row < valid ? row : valid - 1;
        c.off[gq][j] = (uint32_t)(rr * rowb + col * 16 + 3072 - 1024 * j);
      }
  };
  const uint32_t cdst = (cp_x ? G_TILE : 0) + 8192 * (wave & 3);
  auto issue = [&](const Src& c, int kt, int stage) {
    const char* src = c.p + kt * (GBK * 2);
    const uint32_t st = base + stage * G_STAGE + cdst;
    lds_dma_x4(src, c.off[0], st);
    lds_dma_x4(src, c.off[1], st + 4096);
  };

  // per-lane LDS addresses of this wave's operand rows for stage s and
  // k-step ks (first 32-row group; each further group is 4 KiB on, an
  // instruction immediate: the chunk XOR of k_off depends on the row only
  // through bits 1..3), formed once
  uint32_t aad[2][GBK / 16], bad[2][GBK / 16];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      aad[st][ks] = base + st * G_STAGE + (uint32_t)k_off<64>(wn * 128 + l32, 2 * ks + hf);
      bad[st][ks] = base + st * G_STAGE + (uint32_t)(G_TILE + k_off<64>(wm * 32 * WTM + l32, 2 * ks + hf));
    }

  // The tile's 256 bias values go to LDS slice `buf` with its first k-tile
  // (wave 0, two 256-byte copies; columns past N re-read the last one), so
  // the epilogue reads them from LDS: a register load of the bias there
  // would make the compiler wait for every vector memory operation in flight
  // (the next tile's copies, the previous stores) before each use.
  auto issue_bias = [&](int bn0, int buf) {
    if (wave != 0) return;
    const int last = (g.n - bn0 < GBN ? g.n - bn0 : GBN) * 2 - 4;  // byte offset of the last dword in range
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = 4 * lane + 256 * j;
      lds_dma4((const char*)(g.bias + bn0), (uint32_t)(o < last ? o : last), base + G_BIAS + 512 * buf + 256 * j);
    }
  };

  int64_t m0;
  int n0;
  if (!tile_of(0, m0, n0)) return;
  Src cur;
  src_of(m0, n0, cur);
  issue(cur, 0, 0);
  issue_bias(n0, 0);
  for (int64_t it = 0;; ++it) {
    f32x16 acc[WTN][WTM];
#pragma unroll
    for (int ni = 0; ni < WTN; ++ni)
#pragma unroll
      for (int mi = 0; mi < WTM; ++mi) acc[ni][mi] = f32x16{};
    // operand buffers of two k-steps: k-step ks+1's are read while k-step
    // ks's products run
    bf16x8 af[2][WTN], bfr[2][WTM];
    auto load = [&](int buf, int stage, int ks) {
#pragma unroll
      for (int ni = 0; ni < WTN; ++ni) af[buf][ni] = *(lds_bf16x8*)(size_t)(aad[stage][ks] + ni * 4096);
#pragma unroll
      for (int mi = 0; mi < WTM; ++mi) bfr[buf][mi] = *(lds_bf16x8*)(size_t)(bad[stage][ks] + mi * 4096);
    };
    wait_vm<0>();  // this tile's first k-tile landed
    wg_barrier();
    load(0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // one k-tile from stage `stage` (a literal at both call sites), with the
    // copy of the next k-tile into the other stage in flight.  Its first
    // operands are in buffer 0 on entry.  After the last k-step's operands
    // are read, the wave waits for its reads and copies and meets the others
    // at the barrier (every read of this stage done, the next stage landed),
    // then reads the next k-tile's first operands under the last k-step's
    // products.
    auto ktile = [&](int kt, int stage) {
      if (kt + 1 < nk) issue(cur, kt + 1, stage ^ 1);
#pragma unroll
      for (int ks = 0; ks < GBK / 16; ++ks) {
        const int cb = ks & 1;
        if (ks + 1 < GBK / 16) {
          load(cb ^ 1, stage, ks + 1);  // issued before this step's products
        } else {
          __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
          wg_barrier();
          if (kt + 1 < nk) load(cb ^ 1, stage ^ 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ni = 0; ni < WTN; ++ni)
#pragma unroll
          for (int mi = 0; mi < WTM; ++mi)
            acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][ni], bfr[cb][mi], acc[ni][mi], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int kt = 0; kt < nk; kt += 2) {
      ktile(kt, 0);
      if (kt + 1 < nk) ktile(kt + 1, 1);
    }

    // Both stages are free here (every read of them was consumed before the
    // last k-tile's barrier, and no copy is in flight), so the next tile's
    // first k-tile is copied into stage 0 beside this tile's epilogue.
    const int64_t tm0 = m0;
    const int tn0 = n0;
    const bool more = tile_of(it + 1, m0, n0);
    if (more) {
      src_of(m0, n0, cur);
      issue(cur, 0, 0);
      issue_bias(n0, (int)((it + 1) & 1));
    }

    // epilogue: element i of acc[ni][mi] is column n0 + 128 wn + 32 ni +
    // 8 (i>>2) + (i&3) + 4 hf of row m0 + 32 WTM wm + 32 mi + l32.  After bias
    // (and GELU) and the bf16 rounding, the two lanes of a row (hf = 0, 1)
    // trade halves with permlane32 swaps so that each holds 8 consecutive
    // columns per store: hf 0 columns 8q..8q+7 for q = 0, 1; hf 1 for q = 2, 3.
    const uint32_t bslice = base + G_BIAS + 512 * (uint32_t)(it & 1);  // this tile's bias in LDS
  #pragma unroll
    for (int mi = 0; mi < WTM; ++mi) {
      const int64_t m = tm0 + wm * 32 * WTM + mi * 32 + l32;
  #pragma unroll
      for (int ni = 0; ni < WTN; ++ni) {
        const int nb = tn0 + wn * 128 + ni * 32;  // N is a multiple of 64: a 32-column group is all in or all out
        if (nb >= g.n) continue;
        uint32_t d[4][2];
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4 bb =
              *(lds_bf16x4*)(size_t)(bslice + (uint32_t)(wn * 128 + ni * 32 + 8 * q + 4 * hf) * 2);
          float v[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = acc[ni][mi][4 * q + j] + (float)bb[j];
            if (GELU) v[j] = gelu_tanh(v[j]);
          }
          const bf16x2 lo = {(__bf16)v[0], (__bf16)v[1]};
          const bf16x2 hi = {(__bf16)v[2], (__bf16)v[3]};
          d[q][0] = __builtin_bit_cast(uint32_t, lo);
          d[q][1] = __builtin_bit_cast(uint32_t, hi);
        }
  #pragma unroll
        for (int q = 0; q < 2; ++q)
  #pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            // (vdst = group q, vsrc = group q+2; the upper lanes of vdst trade
            // with the lower lanes of vsrc): lanes 0-31 end with their own q
            // in d[q] and the upper lanes' q in d[q+2]; lanes 32-63 with the
            // lower lanes' q+2 in d[q] and their own q+2 in d[q+2]
            const auto r = __builtin_amdgcn_permlane32_swap(d[q][h2], d[q + 2][h2], false, false);
            d[q][h2] = r[0];
            d[q + 2][h2] = r[1];
          }
        if (m < g.m) {
          __bf16* crow = g.c + m * g.ldc + nb;
  #pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int qq = hf ? q + 2 : q;
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            // columns 8 qq + 0..3 sit in d[q], 8 qq + 4..7 in d[q+2], on both halves
            const u32x4 w = u32x4{d[q][0], d[q][1], d[q + 2][0], d[q + 2][1]};
            *(u32x4*)(crow + 8 * qq) = w;
          }
        }
      }
    }
    if (!more) break;
  }
}

}  // namespace

hipError_t launch_gemm_bt(const GemmArgs& g, hipStream_t s) {
  static bool attr_done = false;  // the attribute is idempotent
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bt_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G_LDS);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)gemm_bt_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, G_LDS);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int64_t work = ((g.m + GBM - 1) / GBM) * ((g.n + GBN - 1) / GBN);
  if (work == 0 || g.k == 0) return hipSuccess;
  // one persistent workgroup per CU (128 KiB of LDS each), at most one per
  // tile; a multiple of 8 so that every XCD gets the same number
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  const int64_t want = ((work + 7) / 8) * 8;
  const int64_t cap = (cus / 8 > 0 ? cus / 8 : 1) * 8;
  const dim3 grid((unsigned)(want < cap ? want : cap));
  if (g.gelu)
    hipLaunchKernelGGL(gemm_bt_kernel<true>, grid, dim3(kGThreads), G_LDS, s, g);
  else
    hipLaunchKernelGGL(gemm_bt_kernel<false>, grid, dim3(kGThreads), G_LDS, s, g);
  return hipGetLastError();
}

}  // namespace ra
