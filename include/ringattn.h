/*
 * ringattn.h - C ABI of the gfx950 (MI355X) library for one device's share of
 * exact ring attention.
 *
 * What is computed.  A device holds a local query chunk and receives the key /
 * value blocks of the sequence one at a time in ring order ("Ring Attention:
 * Train 1M Tokens on 8GB GPUs in 2026", section "Ring Attention: Partition
 * Sequence Length, Not Batch").  Each block is attended blockwise while the
 * next one is in flight ("Ring Attention with Blockwise Transformers for
 * Near-Infinite Context", Abstract), and the partial results are merged
 * through the state triple named in the "Gotchas and Failure Modes" section of
 * "Ring Attention: Train 1M Tokens on 8GB GPUs in 2026": running max m,
 * running sum l and unnormalised output acc.  After the last block the output is softmax(Q K^T * scale) V over every
 * visible key (the attention equation of the section "Why Standard Attention
 * Explodes Past 100K Tokens", scale = 1/sqrt(d)) and LSE is its natural-log
 * log-sum-exp.  The merge is the exact online-softmax rule (Milakov and
 * Gimelshein, "Online normalizer calculation for softmax", cited in the arXiv
 * record's reference list), so the result does not depend on block order up
 * to rounding.
 *
 * Tensors and layout.
 *   Q, every K/V block and O are [B, S, H, D] with element strides
 *   (stride_b, stride_s, stride_h) and unit stride along D.  Query row r sits
 *   at global position q_pos0 + r*s; key j of a block at that block's
 *   kv_pos0 + j*s, where s = pos_stride (1 for contiguous chunks; P for the
 *   striped order, in which device i of P holds tokens i, i+P, i+2P, ...).
 *   Causal masking: a key is visible iff its position <= the query's
 *   position (diagonal included).
 *   State: m, l  [B, H, Sq] fp32 contiguous; acc [B, H, Sq, D] fp32
 *   contiguous; m is in natural-log score units, a reference point at or
 *   below the running max of scale * q.k (the kernels move it only when the
 *   sums would grow too large).
 *   LSE [B, H, Sq] fp32 contiguous.  A row that has seen no visible key has
 *   m = -inf, l = 0, acc = 0, and is finalized to O = 0, LSE = -inf.
 *   The state triple is defined up to the choice of m: any (m, l, acc) with
 *   l = sum exp(s - m) and acc = sum exp(s - m) v over the keys seen so far
 *   is a valid state, and acc/l and m + ln l do not depend on that choice.
 *
 * An empty query chunk (q_len = 0) is valid: such a call checks the
 * descriptor, then returns RA_OK without looking at any pointer (empty
 * tensors may have NULL data) and enqueues nothing.
 *
 * Dtypes: (in, out) = (F32, F32), (BF16, BF16) or (BF16, F32).  BF16 inputs
 * use bf16 matrix cores with fp32 accumulation; F32 inputs are computed in
 * fp32 throughout.
 *
 * Ownership and synchronisation.  The caller owns all memory: inputs,
 * outputs, the state workspace and the staging slots.  The library allocates
 * no device memory.  Every call validates its arguments completely before it
 * enqueues anything; on error it returns a non-zero status, enqueues nothing
 * and leaves all buffers untouched, and ringattn_last_error() holds a
 * message for the calling thread.  On success the work is enqueued on the
 * given stream(s) and the call returns without synchronising; results are
 * valid once the compute stream has finished.  Faults inside kernels surface
 * at the caller's next synchronisation.  Nothing throws or aborts across the
 * ABI.  Calls that share buffers on overlapping streams race; calls on
 * disjoint buffers may run concurrently (ringattn_ring_bwd_noalloc excepted:
 * its calls share one device array per GPU).
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RINGATTN_ABI_VERSION 2

typedef enum ra_status {
  RA_OK = 0,
  RA_E_NULL = 1,        /* a required pointer is NULL                           */
  RA_E_SHAPE = 2,       /* negative / inconsistent sizes or strides             */
  RA_E_DTYPE = 3,       /* unsupported (in, out) dtype pair                     */
  RA_E_ALIGN = 4,       /* base pointer or row not 16-byte aligned              */
  RA_E_UNSUPPORTED = 5, /* valid request outside what the kernels implement     */
  RA_E_MEMTYPE = 6,     /* pointer is not the kind of memory the call needs     */
  RA_E_HIP = 7          /* a HIP runtime call failed (message has the HIP text) */
} ra_status;

typedef enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* ring_fwd path selection (ra_desc.flags). */
#define RA_FLAG_PERBLOCK 1 /* force init_state + block_fwd per block + finalize */

typedef struct ra_desc {
  int32_t batch;       /* B >= 1                                              */
  int32_t heads;       /* H >= 1 (key/value heads equal query heads)          */
  int32_t head_dim;    /* D: 64 or 128                                        */
  int32_t causal;      /* 1: key visible iff kv_pos <= q_pos; 0: all visible   */
  int64_t q_len;       /* Sq >= 0: rows of the local query chunk              */
  int64_t kv_len;      /* Ck >= 0: key capacity of a KV block, < 2^30         */
  int64_t q_pos0;      /* global position of query row 0 (q_idx * Sq)         */
  float scale;         /* softmax temperature; <= 0 selects 1/sqrt(D)         */
  int32_t in_dtype;    /* ra_dtype of Q, K, V                                 */
  int32_t out_dtype;   /* ra_dtype of O                                       */
  int32_t flags;       /* RA_FLAG_*                                           */
  int64_t q_stride[3]; /* element strides of Q along (b, s, h)                */
  int64_t kv_stride[3];/* element strides of every K and V block; (s) >= D   */
  int64_t o_stride[3]; /* element strides of O                                */
  int64_t pos_stride;  /* position step between rows and between keys; 0 or 1:
                          contiguous, P: striped order over P devices          */
} ra_desc;

/* Block classes returned by ringattn_block_class. */
#define RA_BLOCK_SKIP 0 /* causal and no key of the block is visible to any row */
#define RA_BLOCK_FULL 1 /* every key visible to every row                       */
#define RA_BLOCK_DIAG 2 /* some keys visible to some rows: masked per element   */

/* Maximum number of device-resident blocks one fused launch carries; longer
 * rings are processed in segments of this many blocks with the state kept in
 * the caller's workspace between segments. */
#define RA_FUSED_MAX_BLOCKS 64

int ringattn_abi_version(void);
/* Fixed text naming a status (never NULL; "unknown status" for values outside
 * ra_status). */
const char* ringattn_status_str(ra_status status);
/* Detail of the last failing call on this thread ("" if none). */
const char* ringattn_last_error(void);

/* Ring schedule of "Ring Attention: Train 1M Tokens on 8GB GPUs in 2026",
 * section "Ring Attention: Partition
 * Sequence Length, Not Batch": at step s the device at ring index q_idx holds
 * the block that started on device (q_idx - s) mod P.  Writes that block index
 * for s = 0..P-1 into order[P] (host memory).  Host only. */
ra_status ringattn_ring_order(int32_t q_idx, int32_t num_devices, int32_t* order);

/* Causal class of the block of kv_len keys starting at kv_pos0 with respect to
 * the query chunk of desc (RA_BLOCK_*), positions stepping by pos_stride;
 * non-causal descriptors give RA_BLOCK_FULL for a non-empty block.  Empty
 * chunks or blocks give RA_BLOCK_SKIP.  Host only; returns -1 for a NULL desc
 * or a negative pos_stride. */
int32_t ringattn_block_class(const ra_desc* desc, int64_t kv_pos0);

/* Start a ring pass: m = -inf, l = 0, acc = 0, the empty state of the triple
 * (running max, running sum, unnormalised output) that "Ring Attention: Train
 * 1M Tokens on 8GB GPUs in 2026", section "Gotchas and Failure Modes", says
 * each device must carry across chunks.  m, l [B, H, Sq] and acc [B, H, Sq, D]
 * are fp32 device memory owned by the caller (layouts above); all three are
 * overwritten.  Errors: RA_E_NULL / RA_E_ALIGN for a missing or misaligned
 * pointer, RA_E_MEMTYPE if one is not device memory, RA_E_HIP if the launch
 * fails; nothing is written then. */
ra_status ringattn_init_state(const ra_desc* desc, float* m, float* l, float* acc, hipStream_t stream);

/* One step of the ring ("Ring Attention: Train 1M Tokens on 8GB GPUs in
 * 2026", section "Ring Attention: Partition Sequence Length, Not Batch":
 * each device attends its query chunk to the block it holds at that step):
 * attend q to one KV block (device pointers k, v whose kv_len keys sit at
 * kv_pos0 + j*pos_stride) and fold the result into (m, l, acc) by the
 * online-softmax rule, which keeps the triple of section "Gotchas and
 * Failure Modes" of the same page exact across chunks whose maxima differ.
 * q, k, v are read only; m, l, acc are read and rewritten in place (caller
 * owned, the state of the previous steps).  A block with fewer valid keys is
 * passed with kv_len set to that count.  A block with no key visible to any
 * row enqueues nothing and returns RA_OK.  Errors as for init_state, plus
 * RA_E_SHAPE / RA_E_DTYPE / RA_E_UNSUPPORTED for a descriptor outside the
 * contract; the state is untouched then. */
ra_status ringattn_block_fwd(const ra_desc* desc, const void* q, const void* k, const void* v, int64_t kv_pos0,
                             float* m, float* l, float* acc, hipStream_t stream);

/* End a ring pass: O = acc / l in out_dtype (0 where l = 0), the
 * softmax(Q K^T * scale) V of the equation in section "Why Standard Attention
 * Explodes Past 100K Tokens" of "Ring Attention: Train 1M Tokens on 8GB GPUs
 * in 2026" over every key the state has seen, and LSE = m + ln l (-inf where
 * l = 0; the log-sum-exp is not on the pages: natural log, fp32 [B, H, Sq]).
 * m, l, acc are read only; o (desc->out_dtype, o_stride) and lse are written.
 * Errors as for init_state. */
ra_status ringattn_finalize(const ra_desc* desc, const float* m, const float* l, const float* acc, void* o,
                            float* lse, hipStream_t stream);

/* Whole ring pass over num_blocks >= 0 blocks given in processing (ring) order:
 * k_blocks[i], v_blocks[i] hold the keys at kv_pos0[i] + j*pos_stride.
 * kv_valid: NULL when every block holds kv_len keys; otherwise block i holds
 * kv_valid[i] valid keys (0 <= kv_valid[i] <= kv_len) at its start and the
 * rest of its kv_len rows is padding, never attended (per-block valid
 * lengths: chunks of unequal length, as the FAQ of "Ring Attention: Train 1M
 * Tokens on 8GB GPUs in 2026" describes, without padded work).  The arrays
 * k_blocks, v_blocks, kv_pos0, kv_valid are host memory.  Equivalent to
 * init_state, block_fwd for each block in array order (with kv_len =
 * kv_valid[i]), finalize, up to rounding: the fused path keeps the state on
 * chip, and the per-block path (resident or streamed) processes the first
 * two blocks that some row can see in four pieces of whole 64-key tiles each,
 * so that a streamed piece is computed while the next one is copied.  The
 * two per-block paths give bitwise-equal results.
 *
 * kv_on_host = 0: blocks are device memory.  Unless flags has
 *   RA_FLAG_PERBLOCK, a fused kernel runs (m, l, acc may be NULL when
 *   num_blocks <= RA_FUSED_MAX_BLOCKS; otherwise they are required).
 * kv_on_host = 1: blocks are pinned host memory (hipHostMalloc'd or
 *   registered), each block densely packed [B, Ck, H, D].  stage_k[0..1] and
 *   stage_v[0..1] are four device slots of B*Ck*H*D elements each; block i is
 *   copied into slot i%2 (its valid rows, piece by piece) with
 *   hipMemcpyAsync / hipMemcpy2DAsync on `copy` while the piece or block
 *   before it is computed on `compute`; events order each piece's copy before
 *   its kernel and a block's kernels before the slot's next copy.  m, l, acc are
 *   required.  `copy` must differ from `compute`.  The host blocks must stay
 *   alive and unchanged until the compute stream has finished.
 * O and LSE are written on `compute`. */
ra_status ringattn_ring_fwd(const ra_desc* desc, const void* q, const void* const* k_blocks,
                            const void* const* v_blocks, const int64_t* kv_pos0, const int64_t* kv_valid,
                            int32_t num_blocks,
                            int32_t kv_on_host, void* const* stage_k, void* const* stage_v, float* m, float* l,
                            float* acc, void* o, float* lse, hipStream_t compute, hipStream_t copy);

/* ---- Backward pass (bf16 inputs only; F32 descriptors give RA_E_UNSUPPORTED).
 * The exact gradient of the output above, the reading taken because the
 * pages train through the ring ("Ring Attention: Train 1M Tokens on 8GB GPUs
 * in 2026", sections "Training Speed: The Numbers" and "Gotchas and Failure
 * Modes") without writing the backward out.  dout (the upstream gradient of
 * O) has Q's layout, strides and dtype; lse is the forward's LSE.  dq is
 * [B, Sq, H, D] and each block's dk, dv [B, kv_len, H, D], fp32, contiguous.
 * A device computes dQ of its chunk and, for every block it receives, its
 * contribution to that block's dK and dV, which in the ring travel on with
 * the block and add up across devices. */

/* delta[b, h, r] = sum_d dout[b, r, h, d] * o[b, r, h, d] (fp32 [B, H, Sq]; o in
 * out_dtype with o_stride). */
ra_status ringattn_bwd_delta(const ra_desc* desc, const void* o, const void* dout, float* delta, hipStream_t stream);

/* One block: dq += this block's part of dQ; dk += and dv += this chunk's
 * contribution (the block's kv_len keys at kv_pos0 + j*pos_stride).  A block
 * with no key visible to any row enqueues nothing and returns RA_OK. */
ra_status ringattn_block_bwd(const ra_desc* desc, const void* q, const void* k, const void* v, int64_t kv_pos0,
                             const void* dout, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                             hipStream_t stream);

/* Whole ring backward on `stream`: delta (into the caller's [B, H, Sq] fp32
 * workspace), dq = 0, then block_bwd for every block (kv_valid as in
 * ringattn_ring_fwd).  dk_blocks[i] and dv_blocks[i] are accumulated into
 * (+=): zero them for the first device of the ring.  Host arrays: k_blocks,
 * v_blocks, kv_pos0, kv_valid, dk_blocks, dv_blocks. */
ra_status ringattn_ring_bwd(const ra_desc* desc, const void* q, const void* const* k_blocks,
                            const void* const* v_blocks, const int64_t* kv_pos0, const int64_t* kv_valid,
                            int32_t num_blocks, const void* o, const void* dout, const float* lse, float* delta,
                            float* dq, float* const* dk_blocks, float* const* dv_blocks, hipStream_t stream);

/* ringattn_ring_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and arguments without the delta
 * workspace.  Its [B, H, Sq] fp32 delta lives in a file-scope device array of
 * RINGATTN_NOALLOC_MAX_ROWS floats (16 MiB) that the library holds on each GPU
 * it runs on until the process ends; the call itself makes no allocation.
 * batch * heads * q_len above RINGATTN_NOALLOC_MAX_ROWS gives
 * RA_E_UNSUPPORTED before anything is enqueued.  All calls on one GPU share
 * that array (each call overwrites it before reading it): calls that overlap
 * on one GPU, on any streams, race. */
#define RINGATTN_NOALLOC_MAX_ROWS (4 << 20)
ra_status ringattn_ring_bwd_noalloc(const ra_desc* desc, const void* q, const void* const* k_blocks,
                                    const void* const* v_blocks, const int64_t* kv_pos0, const int64_t* kv_valid,
                                    int32_t num_blocks, const void* o, const void* dout, const float* lse, float* dq,
                                    float* const* dk_blocks, float* const* dv_blocks, hipStream_t stream);

/* ---- Blockwise feedforward ("Ring Attention with Blockwise Transformers for
 * Near-Infinite Context", Abstract: blockwise computation of self-attention
 * and feedforward).  The pages do not write the network out; the reading
 * taken is the position-wise y = gelu(x W1^T + b1) W2^T + b2 with the tanh
 * form of GELU (Hendrycks and Gimpel), as in GPT-style language models such
 * as the 1.3B model (hidden dim 2048) of "Ring Attention: Train 1M Tokens on
 * 8GB GPUs in 2026", section "Memory Breakdown: 512K Tokens on 4x RTX 3090".
 *
 * All tensors bf16, row-major: x [rows, d_model] (row stride x_stride), W1
 * [d_ff, d_model] and W2 [d_model, d_ff] dense (rows are output features, as
 * in a Linear layer), b1 [d_ff], b2 [d_model], y [rows, d_model] (row stride
 * y_stride).  The rows are processed in blocks of block_rows: per block the
 * hidden activation (fp32-accumulated, GELU applied, rounded to bf16) is
 * written to `workspace`, [block_rows, d_ff] bf16 dense, caller-owned device
 * memory, then multiplied by W2.  The result does not depend on block_rows
 * (each row's arithmetic is the same in any block).  For a chunk in the
 * attention layout [B, S, H, D] with B = 1, x is that tensor with d_model =
 * H*D and x_stride = H*D. */
typedef struct ra_ffn_desc {
  int64_t rows;       /* tokens of the chunk, >= 0                             */
  int32_t d_model;    /* d: a multiple of 64, <= 16384                         */
  int32_t d_ff;       /* F: a multiple of 64, <= 65536                         */
  int64_t x_stride;   /* elements between rows of x: >= d_model, multiple of 8 */
  int64_t y_stride;   /* elements between rows of y: >= d_model, multiple of 8 */
  int64_t block_rows; /* rows per block (>= 1); workspace holds block_rows*d_ff */
} ra_ffn_desc;

/* y = feedforward(x), block by block, enqueued on `stream`.  rows = 0 checks
 * the descriptor and enqueues nothing.  Pointers are device memory, 16-byte
 * aligned; y must not overlap x, the weights or the workspace. */
ra_status ringattn_ffn_fwd(const ra_ffn_desc* desc, const void* x, const void* w1, const void* b1, const void* w2,
                           const void* b2, void* y, void* workspace, hipStream_t stream);

/* Measurement helper, not part of the attention path: a plain device-to-device
 * copy kernel of `bytes` (multiple of 16, 16-byte aligned pointers), used to
 * calibrate hardware byte counters and HBM bandwidth. */
ra_status ringattn_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* Measurement helper, not part of the attention path: `workgroups` groups of
 * 512 threads each issue 4 * iters back-to-back bf16 MFMA products
 * (v_mfma_f32_32x32x16_bf16, 32768 flop each) with no memory traffic, then
 * write one float per thread to `out` (device memory, workgroups * 512
 * floats).  Timed by the caller, it measures the bf16 MFMA rate the part
 * sustains under load. */
ra_status ringattn_probe_mfma(float* out, int32_t workgroups, int32_t iters, hipStream_t stream);

/* Measurement helper, not part of the attention path: the same probe with its
 * operands read once per thread from `operands` (device memory, 16-byte
 * aligned, workgroups * 512 * 32 bf16 values: four 8-element fragments per
 * thread, thread-major) instead of a fixed pattern of small values.  With
 * random bf16 operands, as the attention and feedforward products see, the
 * part draws more power per product and holds a lower clock, so this gives
 * the bf16 MFMA rate it sustains on such data.  Errors: RA_E_NULL, RA_E_SHAPE
 * (the ranges of ringattn_probe_mfma), RA_E_ALIGN, RA_E_MEMTYPE. */
ra_status ringattn_probe_mfma_data(const void* operands, float* out, int32_t workgroups, int32_t iters,
                                   hipStream_t stream);

/* Measurement helper, not part of the attention path: the probe with random
 * operands (the layout of ringattn_probe_mfma_data) where every product's
 * first operand is read from LDS.  Each workgroup copies its 32 KiB of
 * operands twice into a 64 KiB LDS image; per iteration each wave reads
 * `lds_reads` 16-byte-per-lane fragments (1 KiB each) from rotating windows
 * of it and issues 16 products (16 * iters per wave in all), each fragment
 * the first operand of 16 / lds_reads of them.  lds_reads = 16 moves 1 KiB of
 * LDS per product and wave, the ratio of a kernel that reads both operands'
 * tiles from LDS once per product (the forward's K and V^T fragments).  It
 * gives the bf16 MFMA rate the part holds with that LDS traffic beside the
 * matrix cores.  Errors: RA_E_NULL, RA_E_ALIGN, RA_E_SHAPE (workgroups in
 * [1, 65536], iters in [1, 2^22], lds_reads not 4, 8 or 16), RA_E_MEMTYPE. */
ra_status ringattn_probe_mfma_lds(const void* operands, float* out, int32_t workgroups, int32_t iters,
                                  int32_t lds_reads, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
