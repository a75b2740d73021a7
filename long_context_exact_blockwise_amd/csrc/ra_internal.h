// Internal interface between the C-ABI host layer (ringattn_api.hip) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/ringattn.h"

namespace ra {

// Device-resident KV blocks handed to one fused launch, in processing order.
// Passed by value as a kernel argument (fits the kernel-argument segment).
struct BlockTable {
  const void* k[RA_FUSED_MAX_BLOCKS];
  const void* v[RA_FUSED_MAX_BLOCKS];
  int64_t pos0[RA_FUSED_MAX_BLOCKS];  // position of key 0 in row units (contiguous-equivalent, see the API layer)
  int32_t len[RA_FUSED_MAX_BLOCKS];   // valid keys of the block (<= kv_len)
};

// How a launch starts and ends its rows' state.
enum StateMode : int {
  kInitFinalize = 0,  // start from m=-inf,l=0,acc=0; end by writing O and LSE
  kInitStore = 1,     // start from the empty state; end by storing (m,l,acc)
  kLoadStore = 2,     // load (m,l,acc); store it back
  kLoadFinalize = 3,  // load (m,l,acc); end by writing O and LSE
};

struct AttnArgs {
  const void* q;
  void* o;
  float* lse;
  float* m;
  float* l;
  float* acc;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t q_len, kv_len, q_pos0;
  int32_t batch, heads, head_dim, causal, nblocks;
  float scale;        // softmax temperature (natural-log units)
  int32_t out_bf16;   // 1: O is bf16, 0: fp32
};

// One block of the backward pass (bf16 inputs).  Positions are in row units
// (contiguous-equivalent, see the API layer).  dout has q's layout; lse and
// delta are [B, H, Sq] fp32; dq is [B, Sq, H, D] and dk, dv are [B, kv_len, H, D],
// fp32, contiguous, accumulated into (+=).
struct BwdArgs {
  const void* q;
  const void* dout;
  const void* k;
  const void* v;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int64_t q_sb, q_ss, q_sh;
  int64_t kv_sb, kv_ss, kv_sh;
  int64_t q_len, kv_len, q_pos0, kv_pos0;  // kv_len: the block's valid keys; dk/dv rows are kv_cap
  int64_t kv_cap;                          // key capacity of the block (rows of dk, dv)
  int32_t batch, heads, head_dim, causal;
  float scale;
};

// One layer of the blockwise feedforward: C[M, N] = A[M, K] B[N, K]^T +
// bias[N] (then GELU when gelu != 0); bf16, row strides in elements, K a
// multiple of 64.
struct GemmArgs {
  const __bf16* a;
  int64_t lda;
  const __bf16* b;
  int64_t ldb;
  const __bf16* bias;
  __bf16* c;
  int64_t ldc;
  int64_t m;
  int32_t n, k;
  int32_t gelu;
};

// Launchers: validate nothing (the API layer did), enqueue, return the launch
// error (hipSuccess on success).
hipError_t launch_attn_bf16(const AttnArgs& a, const BlockTable& t, int mode, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, const BlockTable& t, int mode, hipStream_t s);
hipError_t launch_init_state(int64_t rows, int32_t d, float* m, float* l, float* acc, hipStream_t s);
hipError_t launch_finalize(const AttnArgs& a, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
// delta[b, h, r] = sum_d dout[b, r, h, d] * o[b, r, h, d]
hipError_t launch_bwd_delta(const AttnArgs& a, const void* dout, float* delta, hipStream_t s);
hipError_t launch_bwd_block(const BwdArgs& a, hipStream_t s);  // launch_bwd_dq, then launch_bwd_dkdv
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s);
hipError_t launch_fill(float* p, int64_t n, hipStream_t s);  // n floats = +0.0f
hipError_t launch_fill_u32(void* p, int64_t n, uint32_t value, hipStream_t s);  // n 32-bit words = value
hipError_t launch_gemm_bt(const GemmArgs& g, hipStream_t s);
hipError_t launch_probe_mfma(const void* src, float* out, int workgroups, int iters, hipStream_t s);
hipError_t launch_probe_mfma_lds(const void* src, float* out, int workgroups, int iters, int lds_reads,
                                 hipStream_t s);

}  // namespace ra
