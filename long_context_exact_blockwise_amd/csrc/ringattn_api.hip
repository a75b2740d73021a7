// C-ABI host layer: argument validation, causal block classification, the
// ring replay driver (fused, per-block, and host-streamed with copy/compute
// overlap) and error reporting.  Every entry point validates completely
// before it enqueues anything and never throws across the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ra_internal.h"

namespace {

using ra::AttnArgs;
using ra::BlockTable;
using ra::BwdArgs;

thread_local std::string g_err;

ra_status fail(ra_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ra_status hip_fail(hipError_t e, const char* what) {
  return fail(RA_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int esize(int32_t dt) { return dt == RA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// True when the rows of D contiguous elements of a [B, S, H, D] tensor with
// element strides st[3] along (b, s, h) are pairwise disjoint: taking the
// dimensions of extent > 1 from the smallest stride up, each stride must
// reach past everything the inner dimensions already span.
bool rows_disjoint(const int64_t st[3], int64_t nb, int64_t ns, int64_t nh, int64_t d) {
  int64_t ext[3] = {nb, ns, nh};
  int idx[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)  // sort the three dims by stride
    for (int j = i + 1; j < 3; ++j)
      if (st[idx[j]] < st[idx[i]]) {
        const int t = idx[i];
        idx[i] = idx[j];
        idx[j] = t;
      }
  int64_t span = d;  // elements [0, span) covered by the inner dims
  for (int i = 0; i < 3; ++i) {
    const int k = idx[i];
    if (ext[k] <= 1) continue;
    if (st[k] < span) return false;
    span = st[k] * (ext[k] - 1) + span;
  }
  return true;
}

// Host-only checks of a descriptor (no HIP calls).
ra_status check_desc(const ra_desc* d) {
  if (!d) return fail(RA_E_NULL, "desc is NULL");
  if (d->batch < 1 || d->heads < 1) return fail(RA_E_SHAPE, "batch (%d) and heads (%d) must be >= 1", d->batch, d->heads);
  if (d->q_len < 0 || d->kv_len < 0)
    return fail(RA_E_SHAPE, "q_len (%lld) and kv_len (%lld) must be >= 0", (long long)d->q_len, (long long)d->kv_len);
  if (d->causal != 0 && d->causal != 1) return fail(RA_E_SHAPE, "causal must be 0 or 1 (got %d)", d->causal);
  if (d->pos_stride < 0) return fail(RA_E_SHAPE, "pos_stride must be >= 0 (got %lld)", (long long)d->pos_stride);
  if (std::isnan(d->scale) || std::isinf(d->scale)) return fail(RA_E_SHAPE, "scale must be finite");
  if ((d->flags & ~RA_FLAG_PERBLOCK) != 0) return fail(RA_E_UNSUPPORTED, "unknown flags 0x%x", d->flags);
  const bool ok_dt = (d->in_dtype == RA_F32 && d->out_dtype == RA_F32) ||
                     (d->in_dtype == RA_BF16 && (d->out_dtype == RA_BF16 || d->out_dtype == RA_F32));
  if (!ok_dt) return fail(RA_E_DTYPE, "unsupported (in, out) dtype pair (%d, %d)", d->in_dtype, d->out_dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  const int64_t* sts[3] = {d->q_stride, d->kv_stride, d->o_stride};
  const char* names[3] = {"q_stride", "kv_stride", "o_stride"};
  const int es[3] = {esize(d->in_dtype), esize(d->in_dtype), esize(d->out_dtype)};
  for (int t = 0; t < 3; ++t) {
    const int64_t dims[3] = {d->batch, t == 1 ? d->kv_len : d->q_len, d->heads};
    for (int i = 0; i < 3; ++i) {
      if (dims[i] > 1 && sts[t][i] <= 0)
        return fail(RA_E_SHAPE, "%s[%d] = %lld must be positive", names[t], i, (long long)sts[t][i]);
      if ((sts[t][i] * es[t]) % 16 != 0)
        return fail(RA_E_ALIGN, "%s[%d] = %lld elements is not a multiple of 16 bytes", names[t], i,
                    (long long)sts[t][i]);
    }
  }
  // Key rows of a block may not overlap (the copies into LDS rely on it).
  if (d->kv_len > 1 && d->kv_stride[1] < d->head_dim)
    return fail(RA_E_SHAPE, "kv_stride[1] (%lld) must be >= head_dim", (long long)d->kv_stride[1]);
  // O is written: no two (b, s, h) rows of D elements may share an element.
  if (!rows_disjoint(d->o_stride, d->batch, d->q_len, d->heads, d->head_dim))
    return fail(RA_E_SHAPE, "o_stride (%lld, %lld, %lld) makes rows of O overlap", (long long)d->o_stride[0],
                (long long)d->o_stride[1], (long long)d->o_stride[2]);
  // The kernels count keys of a block and tiles with 32-bit integers.
  if (d->kv_len >= ((int64_t)1 << 30))
    return fail(RA_E_UNSUPPORTED, "kv_len (%lld) must be below 2^30", (long long)d->kv_len);
  // The kernels address one 64-key tile of a block with 32-bit byte offsets.
  if (d->kv_stride[1] * esize(d->in_dtype) * 64 >= (int64_t)1 << 31)
    return fail(RA_E_UNSUPPORTED, "kv_stride[1] too large (a 64-key tile must span < 2 GiB)");
  return RA_OK;
}

ra_status need_ptr(const void* p, const char* name) {
  if (!p) return fail(RA_E_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(RA_E_ALIGN, "%s is not 16-byte aligned", name);
  return RA_OK;
}

// Memory-kind checks (HIP calls).  want_host: pinned host memory; else device.
ra_status check_mem(const void* p, bool want_host, const char* name) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof attr);
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    if (e == hipErrorInvalidValue)
      return fail(RA_E_MEMTYPE, "%s is not memory known to HIP (pageable host memory?)", name);
    return hip_fail(e, "hipPointerGetAttributes");
  }
  const int t = (int)attr.type;
  if (want_host) {
    if (t != hipMemoryTypeHost) return fail(RA_E_MEMTYPE, "%s must be pinned host memory (type %d)", name, t);
  } else {
    if (t != hipMemoryTypeDevice && t != hipMemoryTypeManaged)
      return fail(RA_E_MEMTYPE, "%s must be device memory (type %d)", name, t);
  }
  return RA_OK;
}

// Positions in row units.  With pos_stride s > 1, row r sits at q_pos0 + r s
// and key j at kv_pos0 + j s; key j is visible to row r iff
// j - r <= floor((q_pos0 - kv_pos0) / s), which is the contiguous rule for a
// query chunk at 0 and a block at -floor((q_pos0 - kv_pos0) / s).  The kernels
// only ever see these contiguous-equivalent positions.
int64_t floor_div(int64_t a, int64_t b) { return a / b - ((a % b != 0) && ((a < 0) != (b < 0))); }
int64_t q_pos_eff(const ra_desc* d) { return d->pos_stride > 1 ? 0 : d->q_pos0; }
// Checking build only (built as a separate library for the tests): before
// each piece's copy into a staging slot, the slot rows it is about to fill are
// set to NaN on the copy stream, so a kernel that reads a slot before its
// copy has landed, or a copy that overwrites a slot still being read, shows
// up as NaN or as a difference from the device-resident pass.
#ifndef RA_POISON_STAGING
#define RA_POISON_STAGING 0
#endif

// Pieces per block for the first two blocks of a per-block ring pass.
#ifndef RA_STREAM_PIECES
#define RA_STREAM_PIECES 4
#endif

int64_t kv_pos_eff(const ra_desc* d, int64_t kv_pos0) {
  return d->pos_stride > 1 ? -floor_div(d->q_pos0 - kv_pos0, d->pos_stride) : kv_pos0;
}

int32_t classify(const ra_desc* d, int64_t kv_pos0, int64_t len) {
  if (d->q_len == 0 || len == 0) return RA_BLOCK_SKIP;
  if (!d->causal) return RA_BLOCK_FULL;
  const int64_t q_first = q_pos_eff(d), q_last = q_first + d->q_len - 1;
  const int64_t k_first = kv_pos_eff(d, kv_pos0), k_last = k_first + len - 1;
  if (k_first > q_last) return RA_BLOCK_SKIP;
  if (k_last <= q_first) return RA_BLOCK_FULL;
  return RA_BLOCK_DIAG;
}

AttnArgs make_args(const ra_desc* d, const void* q, void* o, float* lse, float* m, float* l, float* acc) {
  AttnArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.m = m;
  a.l = l;
  a.acc = acc;
  a.q_sb = d->q_stride[0];
  a.q_ss = d->q_stride[1];
  a.q_sh = d->q_stride[2];
  a.kv_sb = d->kv_stride[0];
  a.kv_ss = d->kv_stride[1];
  a.kv_sh = d->kv_stride[2];
  a.o_sb = d->o_stride[0];
  a.o_ss = d->o_stride[1];
  a.o_sh = d->o_stride[2];
  a.q_len = d->q_len;
  a.kv_len = d->kv_len;
  a.q_pos0 = q_pos_eff(d);
  a.batch = d->batch;
  a.heads = d->heads;
  a.head_dim = d->head_dim;
  a.causal = d->causal;
  a.scale = d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  a.out_bf16 = d->out_dtype == RA_BF16;
  return a;
}

hipError_t launch_attn(const ra_desc* d, AttnArgs a, const BlockTable& t, int nblocks, int mode, hipStream_t s) {
  a.nblocks = nblocks;
  return d->in_dtype == RA_BF16 ? ra::launch_attn_bf16(a, t, mode, s) : ra::launch_attn_f32(a, t, mode, s);
}

ra_status check_state_ptrs(float* m, float* l, float* acc) {
  ra_status st;
  if ((st = need_ptr(m, "m")) != RA_OK) return st;
  if ((st = need_ptr(l, "l")) != RA_OK) return st;
  if ((st = need_ptr(acc, "acc")) != RA_OK) return st;
  return RA_OK;
}

ra_status check_state_mem(float* m, float* l, float* acc) {
  ra_status st;
  if ((st = check_mem(m, false, "m")) != RA_OK) return st;
  if ((st = check_mem(l, false, "l")) != RA_OK) return st;
  if ((st = check_mem(acc, false, "acc")) != RA_OK) return st;
  return RA_OK;
}

// Per-thread events of the host-streamed path, created on first use and kept
// for the life of the thread (not destroyed at exit, when the runtime may
// already be gone).
struct StreamEvents {
  hipEvent_t full[2] = {nullptr, nullptr};
  hipEvent_t free_[2] = {nullptr, nullptr};
  hipEvent_t start = nullptr;
  bool ready = false;
};
thread_local StreamEvents g_ev;

hipError_t events_ready() {
  if (g_ev.ready) return hipSuccess;
  hipError_t e;
  for (int i = 0; i < 2; ++i) {
    if ((e = hipEventCreateWithFlags(&g_ev.full[i], hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&g_ev.free_[i], hipEventDisableTiming)) != hipSuccess) return e;
  }
  if ((e = hipEventCreateWithFlags(&g_ev.start, hipEventDisableTiming)) != hipSuccess) return e;
  g_ev.ready = true;
  return hipSuccess;
}

}  // namespace

// ---- backward helpers ----

namespace {
ra_status check_bwd_desc(const ra_desc* d) {
  ra_status st;
  if ((st = check_desc(d)) != RA_OK) return st;
  if (d->in_dtype != RA_BF16) return fail(RA_E_UNSUPPORTED, "the backward pass takes bf16 inputs");
  if (d->q_stride[1] * 2 * 64 >= (int64_t)1 << 31)
    return fail(RA_E_UNSUPPORTED, "q_stride[1] too large (a 64-row tile must span < 2 GiB)");
  return RA_OK;
}

// ---- the scratch of ringattn_ring_bwd_noalloc ----
// Its per-row delta lives in this file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// the name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns, taken once per device with that device current
// and kept in g_scratch.  Every call on one GPU shares the array; calls that
// overlap on one GPU race.
static __device__ __align__(256) float scratch[RINGATTN_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

ra_status scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = (float*)p;
  }
  *out = g_scratch[dev];
  return RA_OK;
}

BwdArgs make_bwd(const ra_desc* d, const void* q, const void* k, const void* v, int64_t kv_pos0, int64_t valid,
                 const void* dout, const float* lse, const float* delta, float* dq, float* dk, float* dv) {
  BwdArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q;
  a.dout = dout;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.q_sb = d->q_stride[0];
  a.q_ss = d->q_stride[1];
  a.q_sh = d->q_stride[2];
  a.kv_sb = d->kv_stride[0];
  a.kv_ss = d->kv_stride[1];
  a.kv_sh = d->kv_stride[2];
  a.q_len = d->q_len;
  a.kv_len = valid;
  a.kv_cap = d->kv_len;
  a.q_pos0 = q_pos_eff(d);
  a.kv_pos0 = kv_pos_eff(d, kv_pos0);
  a.batch = d->batch;
  a.heads = d->heads;
  a.head_dim = d->head_dim;
  a.causal = d->causal;
  a.scale = d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->head_dim));
  return a;
}
// The ring backward; delta is the caller's workspace, or (use_scratch) the
// library's per-device scratch array.
ra_status ring_bwd(const ra_desc* desc, const void* q, const void* const* k_blocks, const void* const* v_blocks,
                   const int64_t* kv_pos0, const int64_t* kv_valid, int32_t num_blocks, const void* o,
                   const void* dout, const float* lse, float* delta, bool use_scratch, float* dq,
                   float* const* dk_blocks, float* const* dv_blocks, hipStream_t stream) {
  ra_status st;
  if ((st = check_bwd_desc(desc)) != RA_OK) return st;
  if (num_blocks < 0) return fail(RA_E_SHAPE, "num_blocks must be >= 0");
  if (use_scratch && (int64_t)desc->batch * desc->heads * desc->q_len > RINGATTN_NOALLOC_MAX_ROWS)
    return fail(RA_E_UNSUPPORTED, "batch * heads * q_len = %lld exceeds the %d rows of the scratch delta",
                (long long)desc->batch * desc->heads * desc->q_len, RINGATTN_NOALLOC_MAX_ROWS);
  if (desc->q_len == 0) return RA_OK;
  if (num_blocks > 0 && (!k_blocks || !v_blocks || !kv_pos0 || !dk_blocks || !dv_blocks))
    return fail(RA_E_NULL, "k_blocks, v_blocks, kv_pos0, dk_blocks and dv_blocks are required when num_blocks > 0");
  const void* ptrs[] = {q, o, dout, lse, dq, delta};
  const char* names[] = {"q", "o", "dout", "lse", "dq", "delta"};
  const int nptr = use_scratch ? 5 : 6;  // the scratch delta is the library's own
  for (int i = 0; i < nptr; ++i)
    if ((st = need_ptr(ptrs[i], names[i])) != RA_OK) return st;
  auto valid = [&](int i) -> int64_t { return kv_valid ? kv_valid[i] : desc->kv_len; };
  for (int i = 0; i < num_blocks; ++i) {
    if ((st = need_ptr(k_blocks[i], "k_blocks[i]")) != RA_OK) return st;
    if ((st = need_ptr(v_blocks[i], "v_blocks[i]")) != RA_OK) return st;
    if ((st = need_ptr(dk_blocks[i], "dk_blocks[i]")) != RA_OK) return st;
    if ((st = need_ptr(dv_blocks[i], "dv_blocks[i]")) != RA_OK) return st;
    if (valid(i) < 0 || valid(i) > desc->kv_len)
      return fail(RA_E_SHAPE, "kv_valid[%d] = %lld must be in [0, kv_len = %lld]", i, (long long)valid(i),
                  (long long)desc->kv_len);
  }
  for (int i = 0; i < nptr; ++i)
    if ((st = check_mem(ptrs[i], false, names[i])) != RA_OK) return st;
  for (int i = 0; i < num_blocks; ++i) {
    if ((st = check_mem(k_blocks[i], false, "k_blocks[i]")) != RA_OK) return st;
    if ((st = check_mem(v_blocks[i], false, "v_blocks[i]")) != RA_OK) return st;
    if ((st = check_mem(dk_blocks[i], false, "dk_blocks[i]")) != RA_OK) return st;
    if ((st = check_mem(dv_blocks[i], false, "dv_blocks[i]")) != RA_OK) return st;
  }
  if (use_scratch && (st = scratch_address(&delta)) != RA_OK) return st;
  AttnArgs da = make_args(desc, nullptr, (void*)o, nullptr, nullptr, nullptr, nullptr);
  hipError_t e = ra::launch_bwd_delta(da, dout, delta, stream);
  if (e != hipSuccess) return hip_fail(e, "delta launch");
  e = ra::launch_fill(dq, (int64_t)desc->batch * desc->q_len * desc->heads * desc->head_dim, stream);
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  for (int i = 0; i < num_blocks; ++i) {
    if (classify(desc, kv_pos0[i], valid(i)) == RA_BLOCK_SKIP) continue;
    BwdArgs a = make_bwd(desc, q, k_blocks[i], v_blocks[i], kv_pos0[i], valid(i), dout, lse, delta, dq,
                         dk_blocks[i], dv_blocks[i]);
    e = ra::launch_bwd_block(a, stream);
    if (e != hipSuccess) return hip_fail(e, "backward block launch");
  }
  return RA_OK;
}

}  // namespace

extern "C" {

int ringattn_abi_version(void) { return RINGATTN_ABI_VERSION; }

const char* ringattn_status_str(ra_status status) {
  switch (status) {
    case RA_OK: return "RA_OK";
    case RA_E_NULL: return "RA_E_NULL: required pointer is NULL";
    case RA_E_SHAPE: return "RA_E_SHAPE: invalid sizes or strides";
    case RA_E_DTYPE: return "RA_E_DTYPE: unsupported dtype pair";
    case RA_E_ALIGN: return "RA_E_ALIGN: pointer or row not 16-byte aligned";
    case RA_E_UNSUPPORTED: return "RA_E_UNSUPPORTED: outside what the kernels implement";
    case RA_E_MEMTYPE: return "RA_E_MEMTYPE: wrong kind of memory";
    case RA_E_HIP: return "RA_E_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char* ringattn_last_error(void) { return g_err.c_str(); }

ra_status ringattn_ring_order(int32_t q_idx, int32_t num_devices, int32_t* order) {
  g_err.clear();
  if (!order) return fail(RA_E_NULL, "order is NULL");
  if (num_devices < 1) return fail(RA_E_SHAPE, "num_devices must be >= 1");
  if (q_idx < 0 || q_idx >= num_devices) return fail(RA_E_SHAPE, "q_idx must be in [0, num_devices)");
  for (int32_t s = 0; s < num_devices; ++s) order[s] = ((q_idx - s) % num_devices + num_devices) % num_devices;
  return RA_OK;
}

int32_t ringattn_block_class(const ra_desc* desc, int64_t kv_pos0) {
  if (!desc || desc->pos_stride < 0) return -1;
  return classify(desc, kv_pos0, desc->kv_len);
}

ra_status ringattn_init_state(const ra_desc* desc, float* m, float* l, float* acc, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = check_desc(desc)) != RA_OK) return st;
  if (desc->q_len == 0) return RA_OK;  // empty query chunk: nothing to do
  if ((st = check_state_ptrs(m, l, acc)) != RA_OK) return st;
  if ((st = check_state_mem(m, l, acc)) != RA_OK) return st;
  const int64_t rows = (int64_t)desc->batch * desc->heads * desc->q_len;
  hipError_t e = ra::launch_init_state(rows, desc->head_dim, m, l, acc, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "init_state launch");
}

ra_status ringattn_block_fwd(const ra_desc* desc, const void* q, const void* k, const void* v, int64_t kv_pos0,
                             float* m, float* l, float* acc, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = check_desc(desc)) != RA_OK) return st;
  if (desc->q_len == 0 || desc->kv_len == 0) return RA_OK;  // nothing to attend
  if ((st = need_ptr(q, "q")) != RA_OK) return st;
  if ((st = need_ptr(k, "k")) != RA_OK) return st;
  if ((st = need_ptr(v, "v")) != RA_OK) return st;
  if ((st = check_state_ptrs(m, l, acc)) != RA_OK) return st;
  if ((st = check_mem(q, false, "q")) != RA_OK) return st;
  if ((st = check_mem(k, false, "k")) != RA_OK) return st;
  if ((st = check_mem(v, false, "v")) != RA_OK) return st;
  if ((st = check_state_mem(m, l, acc)) != RA_OK) return st;
  if (classify(desc, kv_pos0, desc->kv_len) == RA_BLOCK_SKIP) return RA_OK;
  BlockTable t;
  std::memset(&t, 0, sizeof t);
  t.k[0] = k;
  t.v[0] = v;
  t.pos0[0] = kv_pos_eff(desc, kv_pos0);
  t.len[0] = (int32_t)desc->kv_len;
  AttnArgs a = make_args(desc, q, nullptr, nullptr, m, l, acc);
  hipError_t e = launch_attn(desc, a, t, 1, ra::kLoadStore, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "block kernel launch");
}

ra_status ringattn_finalize(const ra_desc* desc, const float* m, const float* l, const float* acc, void* o,
                            float* lse, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = check_desc(desc)) != RA_OK) return st;
  if (desc->q_len == 0) return RA_OK;  // empty query chunk: nothing to do
  if ((st = check_state_ptrs((float*)m, (float*)l, (float*)acc)) != RA_OK) return st;
  if ((st = need_ptr(o, "o")) != RA_OK) return st;
  if ((st = need_ptr(lse, "lse")) != RA_OK) return st;
  if ((st = check_state_mem((float*)m, (float*)l, (float*)acc)) != RA_OK) return st;
  if ((st = check_mem(o, false, "o")) != RA_OK) return st;
  if ((st = check_mem(lse, false, "lse")) != RA_OK) return st;
  AttnArgs a = make_args(desc, nullptr, o, lse, (float*)m, (float*)l, (float*)acc);
  hipError_t e = ra::launch_finalize(a, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "finalize launch");
}

ra_status ringattn_ring_fwd(const ra_desc* desc, const void* q, const void* const* k_blocks,
                            const void* const* v_blocks, const int64_t* kv_pos0, const int64_t* kv_valid,
                            int32_t num_blocks,
                            int32_t kv_on_host, void* const* stage_k, void* const* stage_v, float* m, float* l,
                            float* acc, void* o, float* lse, hipStream_t compute, hipStream_t copy) {
  g_err.clear();
  ra_status st;
  if ((st = check_desc(desc)) != RA_OK) return st;
  if (num_blocks < 0) return fail(RA_E_SHAPE, "num_blocks must be >= 0");
  if (kv_on_host != 0 && kv_on_host != 1) return fail(RA_E_SHAPE, "kv_on_host must be 0 or 1");
  if (desc->q_len == 0) return RA_OK;  // empty query chunk: nothing to do
  if ((st = need_ptr(q, "q")) != RA_OK) return st;
  if ((st = need_ptr(o, "o")) != RA_OK) return st;
  if ((st = need_ptr(lse, "lse")) != RA_OK) return st;
  if (num_blocks > 0 && (!k_blocks || !v_blocks || !kv_pos0))
    return fail(RA_E_NULL, "k_blocks, v_blocks and kv_pos0 are required when num_blocks > 0");

  // Blocks that some row can see, in the given order.
  auto valid = [&](int i) -> int64_t { return kv_valid ? kv_valid[i] : desc->kv_len; };
  std::vector<int> live;
  live.reserve(num_blocks);
  for (int i = 0; i < num_blocks; ++i) {
    if ((st = need_ptr(k_blocks[i], "k_blocks[i]")) != RA_OK) return st;
    if ((st = need_ptr(v_blocks[i], "v_blocks[i]")) != RA_OK) return st;
    if (valid(i) < 0 || valid(i) > desc->kv_len)
      return fail(RA_E_SHAPE, "kv_valid[%d] = %lld must be in [0, kv_len = %lld]", i, (long long)valid(i),
                  (long long)desc->kv_len);
    if (classify(desc, kv_pos0[i], valid(i)) != RA_BLOCK_SKIP) live.push_back(i);
  }
  const bool perblock = kv_on_host || (desc->flags & RA_FLAG_PERBLOCK);
  const bool needs_ws = perblock || (int)live.size() > RA_FUSED_MAX_BLOCKS;
  if (needs_ws && (st = check_state_ptrs(m, l, acc)) != RA_OK) return st;
  if (kv_on_host) {
    if (!stage_k || !stage_v) return fail(RA_E_NULL, "stage_k and stage_v are required when kv_on_host = 1");
    for (int i = 0; i < 2; ++i) {
      if ((st = need_ptr(stage_k[i], "stage_k[i]")) != RA_OK) return st;
      if ((st = need_ptr(stage_v[i], "stage_v[i]")) != RA_OK) return st;
    }
    if (copy == compute) return fail(RA_E_SHAPE, "copy stream must differ from the compute stream");
    const int64_t hd = (int64_t)desc->heads * desc->head_dim;
    if (desc->kv_stride[2] != desc->head_dim || desc->kv_stride[1] != hd ||
        (desc->batch > 1 && desc->kv_stride[0] != desc->kv_len * hd))
      return fail(RA_E_UNSUPPORTED, "host-resident blocks must be densely packed [B, Ck, H, D]");
  }

  // Memory kinds (HIP).
  if ((st = check_mem(q, false, "q")) != RA_OK) return st;
  if ((st = check_mem(o, false, "o")) != RA_OK) return st;
  if ((st = check_mem(lse, false, "lse")) != RA_OK) return st;
  if (needs_ws && (st = check_state_mem(m, l, acc)) != RA_OK) return st;
  for (int i : live) {
    if ((st = check_mem(k_blocks[i], kv_on_host == 1, "k_blocks[i]")) != RA_OK) return st;
    if ((st = check_mem(v_blocks[i], kv_on_host == 1, "v_blocks[i]")) != RA_OK) return st;
  }
  if (kv_on_host) {
    for (int i = 0; i < 2; ++i) {
      if ((st = check_mem(stage_k[i], false, "stage_k[i]")) != RA_OK) return st;
      if ((st = check_mem(stage_v[i], false, "stage_v[i]")) != RA_OK) return st;
    }
  }

  AttnArgs a = make_args(desc, q, o, lse, m, l, acc);
  BlockTable t;
  std::memset(&t, 0, sizeof t);
  hipError_t e;
  const int64_t rows = (int64_t)desc->batch * desc->heads * desc->q_len;

  if (!perblock) {
    // Fused: state on chip for up to RA_FUSED_MAX_BLOCKS blocks per launch.
    const int nlive = (int)live.size();
    if (nlive <= RA_FUSED_MAX_BLOCKS) {
      for (int j = 0; j < nlive; ++j) {
        t.k[j] = k_blocks[live[j]];
        t.v[j] = v_blocks[live[j]];
        t.pos0[j] = kv_pos_eff(desc, kv_pos0[live[j]]);
        t.len[j] = (int32_t)valid(live[j]);
      }
      e = launch_attn(desc, a, t, nlive, ra::kInitFinalize, compute);
      return e == hipSuccess ? RA_OK : hip_fail(e, "fused kernel launch");
    }
    for (int s0 = 0; s0 < nlive; s0 += RA_FUSED_MAX_BLOCKS) {
      const int n = (nlive - s0 < RA_FUSED_MAX_BLOCKS) ? nlive - s0 : RA_FUSED_MAX_BLOCKS;
      for (int j = 0; j < n; ++j) {
        t.k[j] = k_blocks[live[s0 + j]];
        t.v[j] = v_blocks[live[s0 + j]];
        t.pos0[j] = kv_pos_eff(desc, kv_pos0[live[s0 + j]]);
        t.len[j] = (int32_t)valid(live[s0 + j]);
      }
      const bool first = s0 == 0, last = s0 + n >= nlive;
      const int mode = first ? ra::kInitStore : (last ? ra::kLoadFinalize : ra::kLoadStore);
      e = launch_attn(desc, a, t, n, mode, compute);
      if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
    }
    return RA_OK;
  }

  // Per-block: init, launches with the state in HBM, finalize.  The first
  // two live blocks go in RA_STREAM_PIECES pieces of whole tiles, the rest
  // whole: when the blocks stream from host memory, the kernel of a piece
  // then starts as soon as that piece has landed, and the next piece's copy
  // runs beside it.  Only the first piece's copy is exposed; it was a whole
  // block before.  Both per-block paths split the same way, so they stay
  // bitwise equal.  Pieces that no row can see are skipped.
  e = ra::launch_init_state(rows, desc->head_dim, m, l, acc, compute);
  if (e != hipSuccess) return hip_fail(e, "init_state launch");
  const int64_t q_last_eff = q_pos_eff(desc) + desc->q_len - 1;
  auto piece_rows = [&](size_t s, int64_t nv) -> int64_t {
    if (s >= 2 || RA_STREAM_PIECES <= 1) return nv;
    const int64_t per = (nv + RA_STREAM_PIECES - 1) / RA_STREAM_PIECES;
    return (per + 63) / 64 * 64;
  };
  auto piece_live = [&](int i, int64_t r0) {
    return !desc->causal || kv_pos_eff(desc, kv_pos0[i]) + r0 <= q_last_eff;
  };
  const int64_t es = esize(desc->in_dtype);
  if (!kv_on_host) {
    for (size_t s = 0; s < live.size(); ++s) {
      const int i = live[s];
      const int64_t nv = valid(i), per = piece_rows(s, nv);
      for (int64_t r0 = 0; r0 < nv && piece_live(i, r0); r0 += per) {
        const int64_t off = r0 * desc->kv_stride[1] * es;
        t.k[0] = (const char*)k_blocks[i] + off;
        t.v[0] = (const char*)v_blocks[i] + off;
        t.pos0[0] = kv_pos_eff(desc, kv_pos0[i]) + r0;
        t.len[0] = (int32_t)(nv - r0 < per ? nv - r0 : per);
        e = launch_attn(desc, a, t, 1, ra::kLoadStore, compute);
        if (e != hipSuccess) return hip_fail(e, "block kernel launch");
      }
    }
  } else {
    // Two staging slots: block s goes to slot s % 2.  The copy of block s
    // waits until the kernels of block s-2 (same slot) have finished; the
    // kernel of each piece waits until that piece has landed.  Blocks are
    // densely packed [B, Ck, H, D]: a piece is a run of rows in each batch.
    if ((e = events_ready()) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventRecord(g_ev.start, compute)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(copy, g_ev.start, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    const int64_t row_bytes = (int64_t)desc->heads * desc->head_dim * es;
    const int64_t pitch = desc->kv_len * row_bytes;  // one batch of a block
    auto copy_rows = [&](void* dst, const void* src, int64_t r0, int64_t r1) -> hipError_t {
      char* d = (char*)dst + r0 * row_bytes;
      const char* sp = (const char*)src + r0 * row_bytes;
      if (desc->batch == 1) return hipMemcpyAsync(d, sp, (size_t)((r1 - r0) * row_bytes), hipMemcpyHostToDevice, copy);
      return hipMemcpy2DAsync(d, (size_t)pitch, sp, (size_t)pitch, (size_t)((r1 - r0) * row_bytes), (size_t)desc->batch,
                              hipMemcpyHostToDevice, copy);
    };
    for (size_t s = 0; s < live.size(); ++s) {
      const int i = live[s];
      const int slot = (int)(s & 1);
      if (s >= 2 && (e = hipStreamWaitEvent(copy, g_ev.free_[slot], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");
      const int64_t nv = valid(i), per = piece_rows(s, nv);
      for (int64_t r0 = 0; r0 < nv && piece_live(i, r0); r0 += per) {
        const int64_t r1 = nv - r0 < per ? nv : r0 + per;
#if RA_POISON_STAGING
        for (int b = 0; b < desc->batch; ++b)
          for (void* dst : {stage_k[slot], stage_v[slot]})
            if ((e = ra::launch_fill_u32((char*)dst + b * pitch + r0 * row_bytes, (r1 - r0) * row_bytes / 4,
                                         0xFFFFFFFFu, copy)) != hipSuccess)
              return hip_fail(e, "poison launch");
#endif
        if ((e = copy_rows(stage_k[slot], k_blocks[i], r0, r1)) != hipSuccess) return hip_fail(e, "hipMemcpyAsync K");
        if ((e = copy_rows(stage_v[slot], v_blocks[i], r0, r1)) != hipSuccess) return hip_fail(e, "hipMemcpyAsync V");
        if ((e = hipEventRecord(g_ev.full[slot], copy)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        if ((e = hipStreamWaitEvent(compute, g_ev.full[slot], 0)) != hipSuccess)
          return hip_fail(e, "hipStreamWaitEvent");
        t.k[0] = (const char*)stage_k[slot] + r0 * row_bytes;
        t.v[0] = (const char*)stage_v[slot] + r0 * row_bytes;
        t.pos0[0] = kv_pos_eff(desc, kv_pos0[i]) + r0;
        t.len[0] = (int32_t)(r1 - r0);
        e = launch_attn(desc, a, t, 1, ra::kLoadStore, compute);
        if (e != hipSuccess) return hip_fail(e, "block kernel launch");
      }
      if ((e = hipEventRecord(g_ev.free_[slot], compute)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
  }
  e = ra::launch_finalize(a, compute);
  return e == hipSuccess ? RA_OK : hip_fail(e, "finalize launch");
}


ra_status ringattn_bwd_delta(const ra_desc* desc, const void* o, const void* dout, float* delta, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = check_bwd_desc(desc)) != RA_OK) return st;
  if (desc->q_len == 0) return RA_OK;
  const void* ptrs[] = {o, dout, delta};
  const char* names[] = {"o", "dout", "delta"};
  for (int i = 0; i < 3; ++i)
    if ((st = need_ptr(ptrs[i], names[i])) != RA_OK) return st;
  for (int i = 0; i < 3; ++i)
    if ((st = check_mem(ptrs[i], false, names[i])) != RA_OK) return st;
  AttnArgs a = make_args(desc, nullptr, (void*)o, nullptr, nullptr, nullptr, nullptr);
  hipError_t e = ra::launch_bwd_delta(a, dout, delta, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "delta launch");
}

ra_status ringattn_block_bwd(const ra_desc* desc, const void* q, const void* k, const void* v, int64_t kv_pos0,
                             const void* dout, const float* lse, const float* delta, float* dq, float* dk, float* dv,
                             hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = check_bwd_desc(desc)) != RA_OK) return st;
  if (desc->q_len == 0 || desc->kv_len == 0) return RA_OK;
  const void* ptrs[] = {q, k, v, dout, lse, delta, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "dout", "lse", "delta", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i)
    if ((st = need_ptr(ptrs[i], names[i])) != RA_OK) return st;
  for (int i = 0; i < 9; ++i)
    if ((st = check_mem(ptrs[i], false, names[i])) != RA_OK) return st;
  if (classify(desc, kv_pos0, desc->kv_len) == RA_BLOCK_SKIP) return RA_OK;
  BwdArgs a = make_bwd(desc, q, k, v, kv_pos0, desc->kv_len, dout, lse, delta, dq, dk, dv);
  hipError_t e = ra::launch_bwd_block(a, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "backward block launch");
}

ra_status ringattn_ring_bwd(const ra_desc* desc, const void* q, const void* const* k_blocks,
                            const void* const* v_blocks, const int64_t* kv_pos0, const int64_t* kv_valid,
                            int32_t num_blocks, const void* o, const void* dout, const float* lse, float* delta,
                            float* dq, float* const* dk_blocks, float* const* dv_blocks, hipStream_t stream) {
  g_err.clear();
  return ring_bwd(desc, q, k_blocks, v_blocks, kv_pos0, kv_valid, num_blocks, o, dout, lse, delta, false, dq, dk_blocks,
                  dv_blocks, stream);
}

ra_status ringattn_ring_bwd_noalloc(const ra_desc* desc, const void* q, const void* const* k_blocks,
                                    const void* const* v_blocks, const int64_t* kv_pos0, const int64_t* kv_valid,
                                    int32_t num_blocks, const void* o, const void* dout, const float* lse, float* dq,
                                    float* const* dk_blocks, float* const* dv_blocks, hipStream_t stream) {
  g_err.clear();
  return ring_bwd(desc, q, k_blocks, v_blocks, kv_pos0, kv_valid, num_blocks, o, dout, lse, nullptr, true, dq,
                  dk_blocks, dv_blocks, stream);
}

ra_status ringattn_ffn_fwd(const ra_ffn_desc* d, const void* x, const void* w1, const void* b1, const void* w2,
                           const void* b2, void* y, void* workspace, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if (!d) return fail(RA_E_NULL, "desc is NULL");
  if (d->rows < 0 || d->d_model <= 0 || d->d_ff <= 0)
    return fail(RA_E_SHAPE, "rows (%lld) must be >= 0, d_model (%d) and d_ff (%d) > 0", (long long)d->rows,
                d->d_model, d->d_ff);
  if (d->d_model % 64 || d->d_ff % 64)
    return fail(RA_E_UNSUPPORTED, "d_model (%d) and d_ff (%d) must be multiples of 64", d->d_model, d->d_ff);
  if (d->d_model > 16384 || d->d_ff > 65536)
    return fail(RA_E_UNSUPPORTED, "d_model <= 16384 and d_ff <= 65536 (got %d, %d)", d->d_model, d->d_ff);
  if (d->x_stride < d->d_model || d->y_stride < d->d_model)
    return fail(RA_E_SHAPE, "x_stride (%lld) and y_stride (%lld) must be >= d_model", (long long)d->x_stride,
                (long long)d->y_stride);
  if (d->x_stride % 8 || d->y_stride % 8)
    return fail(RA_E_ALIGN, "x_stride and y_stride must be multiples of 8 elements (16-byte rows)");
  if (d->x_stride * 2 * 256 >= (int64_t)1 << 31)
    return fail(RA_E_UNSUPPORTED, "x_stride too large (a 256-row tile must span < 2 GiB)");
  if (d->rows == 0) return RA_OK;
  if (d->block_rows <= 0) return fail(RA_E_SHAPE, "block_rows must be >= 1");
  const void* ptrs[] = {x, w1, b1, w2, b2, y, workspace};
  const char* names[] = {"x", "w1", "b1", "w2", "b2", "y", "workspace"};
  for (int i = 0; i < 7; ++i)
    if ((st = need_ptr(ptrs[i], names[i])) != RA_OK) return st;
  for (int i = 0; i < 7; ++i)
    if ((st = check_mem(ptrs[i], false, names[i])) != RA_OK) return st;
  const int64_t rb = d->block_rows < d->rows ? d->block_rows : d->rows;
  for (int64_t r0 = 0; r0 < d->rows; r0 += rb) {
    const int64_t m = d->rows - r0 < rb ? d->rows - r0 : rb;
    ra::GemmArgs g1{(const __bf16*)x + r0 * d->x_stride, d->x_stride, (const __bf16*)w1, d->d_model,
                    (const __bf16*)b1, (__bf16*)workspace, d->d_ff, m, d->d_ff, d->d_model, 1};
    hipError_t e = ra::launch_gemm_bt(g1, stream);
    if (e != hipSuccess) return hip_fail(e, "feedforward layer 1 launch");
    ra::GemmArgs g2{(const __bf16*)workspace, d->d_ff, (const __bf16*)w2, d->d_ff, (const __bf16*)b2,
                    (__bf16*)y + r0 * d->y_stride, d->y_stride, m, d->d_model, d->d_ff, 0};
    e = ra::launch_gemm_bt(g2, stream);
    if (e != hipSuccess) return hip_fail(e, "feedforward layer 2 launch");
  }
  return RA_OK;
}

ra_status ringattn_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = need_ptr(src, "src")) != RA_OK) return st;
  if ((st = need_ptr(dst, "dst")) != RA_OK) return st;
  if (bytes < 0 || bytes % 16 != 0) return fail(RA_E_SHAPE, "bytes must be a non-negative multiple of 16");
  if ((st = check_mem(src, false, "src")) != RA_OK) return st;
  if ((st = check_mem(dst, false, "dst")) != RA_OK) return st;
  hipError_t e = ra::launch_copy(src, dst, bytes, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "copy launch");
}

ra_status ringattn_probe_mfma(float* out, int32_t workgroups, int32_t iters, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = need_ptr(out, "out")) != RA_OK) return st;
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 24))
    return fail(RA_E_SHAPE, "workgroups must be in [1, 65536] and iters in [1, 2^24]");
  if ((st = check_mem(out, false, "out")) != RA_OK) return st;
  hipError_t e = ra::launch_probe_mfma(nullptr, out, workgroups, iters, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "probe launch");
}

ra_status ringattn_probe_mfma_data(const void* operands, float* out, int32_t workgroups, int32_t iters,
                                   hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = need_ptr(operands, "operands")) != RA_OK) return st;
  if ((st = need_ptr(out, "out")) != RA_OK) return st;
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 24))
    return fail(RA_E_SHAPE, "workgroups must be in [1, 65536] and iters in [1, 2^24]");
  if ((st = check_mem(operands, false, "operands")) != RA_OK) return st;
  if ((st = check_mem(out, false, "out")) != RA_OK) return st;
  hipError_t e = ra::launch_probe_mfma(operands, out, workgroups, iters, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "probe launch");
}

ra_status ringattn_probe_mfma_lds(const void* operands, float* out, int32_t workgroups, int32_t iters,
                                  int32_t lds_reads, hipStream_t stream) {
  g_err.clear();
  ra_status st;
  if ((st = need_ptr(operands, "operands")) != RA_OK) return st;
  if ((st = need_ptr(out, "out")) != RA_OK) return st;
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 22))
    return fail(RA_E_SHAPE, "workgroups must be in [1, 65536] and iters in [1, 2^22]");
  if (lds_reads != 4 && lds_reads != 8 && lds_reads != 16)
    return fail(RA_E_SHAPE, "lds_reads must be 4, 8 or 16 (got %d)", lds_reads);
  if ((st = check_mem(operands, false, "operands")) != RA_OK) return st;
  if ((st = check_mem(out, false, "out")) != RA_OK) return st;
  hipError_t e = ra::launch_probe_mfma_lds(operands, out, workgroups, iters, lds_reads, stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "probe launch");
}

}  // extern "C"
