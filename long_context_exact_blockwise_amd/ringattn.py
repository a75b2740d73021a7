"""ctypes binding over libringattn.so (argument marshalling only).

Functions carry the C entry points' names.  torch tensors supply device
pointers, strides and the current HIP stream; every step of the attention
path runs in the library's kernels.  A missing library raises: there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RINGATTN_LIBRARY may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("RINGATTN_LIBRARY") or os.path.join(_HERE, "libringattn.so")

RA_OK, RA_E_NULL, RA_E_SHAPE, RA_E_DTYPE, RA_E_ALIGN, RA_E_UNSUPPORTED, RA_E_MEMTYPE, RA_E_HIP = range(8)
RA_F32, RA_BF16 = 0, 1
RA_FLAG_PERBLOCK = 1
RA_BLOCK_SKIP, RA_BLOCK_FULL, RA_BLOCK_DIAG = 0, 1, 2
RA_FUSED_MAX_BLOCKS = 64
ABI_VERSION = 2

SYMBOLS = (
    "ringattn_abi_version", "ringattn_status_str", "ringattn_last_error", "ringattn_ring_order",
    "ringattn_block_class", "ringattn_init_state", "ringattn_block_fwd", "ringattn_finalize",
    "ringattn_ring_fwd", "ringattn_probe_copy", "ringattn_bwd_delta", "ringattn_block_bwd", "ringattn_ring_bwd",
    "ringattn_ffn_fwd", "ringattn_probe_mfma", "ringattn_ring_bwd_noalloc", "ringattn_probe_mfma_data",
    "ringattn_probe_mfma_lds",
)
NOALLOC_MAX_ROWS = 4 << 20


class RingAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


class RaDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
        ("q_pos0", ctypes.c_int64), ("scale", ctypes.c_float), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("kv_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("pos_stride", ctypes.c_int64),
    ]


class RaFfnDesc(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("x_stride", ctypes.c_int64), ("y_stride", ctypes.c_int64), ("block_rows", ctypes.c_int64),
    ]


_lib = None


def lib():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path: str):
    """Open a build of the library at `path` and declare its C signatures
    (the functions below call the one lib() returns)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(or python -m long_context_exact_blockwise_amd.build)")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(RaDesc)
    L.ringattn_abi_version.restype = ctypes.c_int
    L.ringattn_status_str.restype = ctypes.c_char_p
    L.ringattn_status_str.argtypes = [ctypes.c_int]
    L.ringattn_last_error.restype = ctypes.c_char_p
    L.ringattn_ring_order.restype = ctypes.c_int
    L.ringattn_ring_order.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    L.ringattn_block_class.restype = ctypes.c_int32
    L.ringattn_block_class.argtypes = [D, ctypes.c_int64]
    L.ringattn_init_state.restype = ctypes.c_int
    L.ringattn_init_state.argtypes = [D, P, P, P, P]
    L.ringattn_block_fwd.restype = ctypes.c_int
    L.ringattn_block_fwd.argtypes = [D, P, P, P, ctypes.c_int64, P, P, P, P]
    L.ringattn_finalize.restype = ctypes.c_int
    L.ringattn_finalize.argtypes = [D, P, P, P, P, P, P]
    L.ringattn_ring_fwd.restype = ctypes.c_int
    L.ringattn_ring_fwd.argtypes = [D, P, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32,
                                    ctypes.POINTER(P), ctypes.POINTER(P), P, P, P, P, P, P, P]
    L.ringattn_probe_copy.restype = ctypes.c_int
    L.ringattn_probe_copy.argtypes = [P, P, ctypes.c_int64, P]
    L.ringattn_bwd_delta.restype = ctypes.c_int
    L.ringattn_bwd_delta.argtypes = [D, P, P, P, P]
    L.ringattn_block_bwd.restype = ctypes.c_int
    L.ringattn_block_bwd.argtypes = [D, P, P, P, ctypes.c_int64, P, P, P, P, P, P, P]
    L.ringattn_probe_mfma.restype = ctypes.c_int
    L.ringattn_probe_mfma.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P]
    L.ringattn_probe_mfma_data.restype = ctypes.c_int
    L.ringattn_probe_mfma_data.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, P]
    L.ringattn_probe_mfma_lds.restype = ctypes.c_int
    L.ringattn_probe_mfma_lds.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    L.ringattn_ffn_fwd.restype = ctypes.c_int
    L.ringattn_ffn_fwd.argtypes = [ctypes.POINTER(RaFfnDesc), P, P, P, P, P, P, P, P]
    L.ringattn_ring_bwd.restype = ctypes.c_int
    L.ringattn_ring_bwd.argtypes = [D, P, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, P, P, P, P, P,
                                    ctypes.POINTER(P), ctypes.POINTER(P), P]
    L.ringattn_ring_bwd_noalloc.restype = ctypes.c_int
    L.ringattn_ring_bwd_noalloc.argtypes = [D, P, ctypes.POINTER(P), ctypes.POINTER(P),
                                            ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                            ctypes.c_int32, P, P, P, P, ctypes.POINTER(P), ctypes.POINTER(P), P]
    if L.ringattn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version mismatch")
    return L


def _check(status: int):
    if status != RA_OK:
        L = lib()
        msg = L.ringattn_last_error().decode() or L.ringattn_status_str(status).decode()
        raise RingAttnError(status, msg)


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return RA_BF16
    if t == torch.float32:
        return RA_F32
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s) -> ctypes.c_void_p:
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(q: torch.Tensor, kv_block: torch.Tensor, o: Optional[torch.Tensor] = None, *, q_pos0: int = 0,
              causal: bool = False, scale: float = 0.0, flags: int = 0, out_dtype=None,
              pos_stride: int = 1) -> RaDesc:
    """Descriptor from tensors in [B, S, H, D] layout (strides taken as given;
    the D stride must be 1).  kv_block is any one KV block (all share strides
    and the key capacity kv_len)."""
    b, sq, h, d = q.shape
    kb, ck, kh, kd = kv_block.shape
    if (kb, kh, kd) != (b, h, d):
        raise ValueError("q and kv blocks must share B, H and D")
    if q.stride(3) != 1 or kv_block.stride(3) != 1 or (o is not None and o.stride(3) != 1):
        raise ValueError("the head_dim axis must be contiguous")
    desc = RaDesc()
    desc.batch, desc.heads, desc.head_dim = b, h, d
    desc.causal = 1 if causal else 0
    desc.q_len, desc.kv_len, desc.q_pos0 = sq, ck, q_pos0
    desc.scale = scale
    desc.in_dtype = _dt(q.dtype)
    if out_dtype is None:
        out_dtype = o.dtype if o is not None else q.dtype
    desc.out_dtype = _dt(out_dtype)
    desc.flags = flags
    desc.pos_stride = pos_stride
    for i in range(3):
        desc.q_stride[i] = q.stride(i)
        desc.kv_stride[i] = kv_block.stride(i)
        desc.o_stride[i] = o.stride(i) if o is not None else q.stride(i)
    return desc


def ringattn_ring_order(q_idx: int, num_devices: int) -> list:
    arr = (ctypes.c_int32 * max(num_devices, 1))()
    _check(lib().ringattn_ring_order(q_idx, num_devices, arr))
    return list(arr)[:num_devices]


def ringattn_block_class(desc: RaDesc, kv_pos0: int) -> int:
    return lib().ringattn_block_class(ctypes.byref(desc), kv_pos0)


def ringattn_init_state(desc: RaDesc, m, l, acc, stream=None):
    _check(lib().ringattn_init_state(ctypes.byref(desc), _ptr(m), _ptr(l), _ptr(acc), _stream(stream)))


def ringattn_block_fwd(desc: RaDesc, q, k, v, kv_pos0: int, m, l, acc, stream=None):
    _check(lib().ringattn_block_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), kv_pos0, _ptr(m), _ptr(l),
                                    _ptr(acc), _stream(stream)))


def ringattn_finalize(desc: RaDesc, m, l, acc, o, lse, stream=None):
    _check(lib().ringattn_finalize(ctypes.byref(desc), _ptr(m), _ptr(l), _ptr(acc), _ptr(o), _ptr(lse),
                                   _stream(stream)))


def ringattn_ring_fwd(desc: RaDesc, q, k_blocks: Sequence, v_blocks: Sequence, kv_pos0: Sequence[int], o, lse,
                      m=None, l=None, acc=None, *, kv_valid: Optional[Sequence[int]] = None, kv_on_host: bool = False,
                      stage_k: Sequence = None, stage_v: Sequence = None, stream=None, copy_stream=None):
    n = len(k_blocks)
    P = ctypes.c_void_p
    kp = (P * max(n, 1))(*[t.data_ptr() for t in k_blocks])
    vp = (P * max(n, 1))(*[t.data_ptr() for t in v_blocks])
    pp = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_pos0])
    nv = None if kv_valid is None else (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_valid])
    sk = sv = None
    if stage_k is not None:
        sk = (P * 2)(*[t.data_ptr() for t in stage_k])
        sv = (P * 2)(*[t.data_ptr() for t in stage_v])
    cs = _stream(copy_stream) if copy_stream is not None else None
    _check(lib().ringattn_ring_fwd(ctypes.byref(desc), _ptr(q), kp, vp, pp, nv, n, 1 if kv_on_host else 0, sk,
                                   sv, _ptr(m), _ptr(l), _ptr(acc), _ptr(o), _ptr(lse), _stream(stream), cs))


def ringattn_probe_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int, stream=None):
    _check(lib().ringattn_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


PROBE_THREADS = 512
PROBE_FLOP_PER_ITER_PER_WAVE = 4 * 32768  # four 32x32x16 products


def ringattn_probe_mfma(out: torch.Tensor, workgroups: int, iters: int, stream=None):
    _check(lib().ringattn_probe_mfma(_ptr(out), workgroups, iters, _stream(stream)))


PROBE_OPERANDS_PER_THREAD = 32  # bf16 values: four 8-element fragments


def ringattn_probe_mfma_data(operands: torch.Tensor, out: torch.Tensor, workgroups: int, iters: int, stream=None):
    _check(lib().ringattn_probe_mfma_data(_ptr(operands), _ptr(out), workgroups, iters, _stream(stream)))


PROBE_LDS_FLOP_PER_ITER_PER_WAVE = 16 * 32768  # sixteen 32x32x16 products


def ringattn_probe_mfma_lds(operands: torch.Tensor, out: torch.Tensor, workgroups: int, iters: int, lds_reads: int,
                            stream=None):
    _check(lib().ringattn_probe_mfma_lds(_ptr(operands), _ptr(out), workgroups, iters, lds_reads,
                                         _stream(stream)))


# ---- convenience wrappers (allocation of outputs / workspace with torch) ----

def state_buffers(desc: RaDesc, device):
    rows = (desc.batch, desc.heads, desc.q_len)
    m = torch.empty(rows, dtype=torch.float32, device=device)
    l = torch.empty(rows, dtype=torch.float32, device=device)
    acc = torch.empty(rows + (desc.head_dim,), dtype=torch.float32, device=device)
    return m, l, acc


def ring_forward(q: torch.Tensor, k_blocks: Sequence[torch.Tensor], v_blocks: Sequence[torch.Tensor],
                 kv_pos0: Sequence[int], *, q_pos0: int = 0, causal: bool = False, scale: float = 0.0,
                 perblock: bool = False, out_dtype=None, o=None, lse=None, workspace=None,
                 kv_valid: Optional[Sequence[int]] = None, pos_stride: int = 1):
    """Attention of q over the blocks (device tensors) in the given order;
    block i contributes its first kv_valid[i] keys (all when kv_valid is
    None).  Returns (O [B, Sq, H, D], LSE [B, H, Sq] fp32)."""
    out_dtype = out_dtype or q.dtype
    b, sq, h, d = q.shape
    if o is None:
        o = torch.empty((b, sq, h, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((b, h, sq), dtype=torch.float32, device=q.device)
    desc = make_desc(q, k_blocks[0] if len(k_blocks) else q, o, q_pos0=q_pos0, causal=causal, scale=scale,
                     flags=RA_FLAG_PERBLOCK if perblock else 0, pos_stride=pos_stride)
    if len(k_blocks) == 0:
        desc.kv_len = 0
    need_ws = perblock or len(k_blocks) > RA_FUSED_MAX_BLOCKS
    m = l = acc = None
    if need_ws:
        m, l, acc = workspace if workspace is not None else state_buffers(desc, q.device)
    ringattn_ring_fwd(desc, q, k_blocks, v_blocks, kv_pos0, o, lse, m, l, acc, kv_valid=kv_valid)
    return o, lse


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# ---- backward ----

def ringattn_bwd_delta(desc: RaDesc, o, dout, delta, stream=None):
    _check(lib().ringattn_bwd_delta(ctypes.byref(desc), _ptr(o), _ptr(dout), _ptr(delta), _stream(stream)))


def ringattn_block_bwd(desc: RaDesc, q, k, v, kv_pos0: int, dout, lse, delta, dq, dk, dv, stream=None):
    _check(lib().ringattn_block_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), kv_pos0, _ptr(dout), _ptr(lse),
                                    _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def ringattn_ring_bwd(desc: RaDesc, q, k_blocks: Sequence, v_blocks: Sequence, kv_pos0: Sequence[int], o, dout, lse,
                      delta, dq, dk_blocks: Sequence, dv_blocks: Sequence, *, kv_valid: Optional[Sequence[int]] = None,
                      stream=None):
    n = len(k_blocks)
    P = ctypes.c_void_p
    arr = lambda ts: (P * max(n, 1))(*[t.data_ptr() for t in ts])  # noqa: E731
    pp = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_pos0])
    nv = None if kv_valid is None else (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_valid])
    _check(lib().ringattn_ring_bwd(ctypes.byref(desc), _ptr(q), arr(k_blocks), arr(v_blocks), pp, nv, n, _ptr(o),
                                   _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), arr(dk_blocks), arr(dv_blocks),
                                   _stream(stream)))


def ringattn_ring_bwd_noalloc(desc: RaDesc, q, k_blocks: Sequence, v_blocks: Sequence, kv_pos0: Sequence[int], o,
                              dout, lse, dq, dk_blocks: Sequence, dv_blocks: Sequence, *,
                              kv_valid: Optional[Sequence[int]] = None, stream=None):
    n = len(k_blocks)
    P = ctypes.c_void_p
    arr = lambda ts: (P * max(n, 1))(*[t.data_ptr() for t in ts])  # noqa: E731
    pp = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_pos0])
    nv = None if kv_valid is None else (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_valid])
    _check(lib().ringattn_ring_bwd_noalloc(ctypes.byref(desc), _ptr(q), arr(k_blocks), arr(v_blocks), pp, nv, n,
                                           _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), arr(dk_blocks), arr(dv_blocks),
                                           _stream(stream)))


def ring_backward(q: torch.Tensor, k_blocks: Sequence[torch.Tensor], v_blocks: Sequence[torch.Tensor],
                  kv_pos0: Sequence[int], o: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, *, q_pos0: int = 0,
                  causal: bool = False, scale: float = 0.0, kv_valid: Optional[Sequence[int]] = None,
                  pos_stride: int = 1):
    """Gradients of one device's ring-attention output (bf16 inputs).  Returns
    (dQ, [dK_i], [dV_i]) fp32 in [B, S, H, D]; dK_i / dV_i are this chunk's
    contributions to block i (allocated zeroed here)."""
    b, sq, h, d = q.shape
    desc = make_desc(q, k_blocks[0] if len(k_blocks) else q, o, q_pos0=q_pos0, causal=causal, scale=scale,
                     pos_stride=pos_stride)
    if len(k_blocks) == 0:
        desc.kv_len = 0
    ck = desc.kv_len
    delta = torch.empty((b, h, sq), dtype=torch.float32, device=q.device)
    dq = torch.empty((b, sq, h, d), dtype=torch.float32, device=q.device)
    dk = [torch.zeros((b, ck, h, d), dtype=torch.float32, device=q.device) for _ in k_blocks]
    dv = [torch.zeros((b, ck, h, d), dtype=torch.float32, device=q.device) for _ in k_blocks]
    ringattn_ring_bwd(desc, q, k_blocks, v_blocks, kv_pos0, o, dout, lse, delta, dq, dk, dv, kv_valid=kv_valid)
    return dq, dk, dv


# ---- blockwise feedforward ----

def ringattn_ffn_fwd(desc: RaFfnDesc, x, w1, b1, w2, b2, y, workspace, stream=None):
    _check(lib().ringattn_ffn_fwd(ctypes.byref(desc), _ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(y),
                                  _ptr(workspace), _stream(stream)))


def ffn_desc(x: torch.Tensor, w1: torch.Tensor, y: Optional[torch.Tensor] = None, block_rows: int = 0) -> RaFfnDesc:
    """Descriptor for x [rows, d_model] (row stride as given, unit column
    stride) and W1 [d_ff, d_model]; block_rows 0 means all rows in one block."""
    rows, d = x.shape
    if x.stride(1) != 1 or (y is not None and y.stride(1) != 1):
        raise ValueError("the feature axis must be contiguous")
    desc = RaFfnDesc()
    desc.rows, desc.d_model, desc.d_ff = rows, d, w1.shape[0]
    desc.x_stride = x.stride(0)
    desc.y_stride = y.stride(0) if y is not None else d
    desc.block_rows = block_rows if block_rows > 0 else max(rows, 1)
    return desc


def ffn_forward(x: torch.Tensor, w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: torch.Tensor, *,
                block_rows: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = gelu(x W1^T + b1) W2^T + b2 over row blocks (bf16).  Allocates y
    and, unless given, the [block_rows, d_ff] workspace."""
    y = torch.empty((x.shape[0], w2.shape[0]), dtype=x.dtype, device=x.device)
    desc = ffn_desc(x, w1, y, block_rows)
    if workspace is None:
        workspace = torch.empty((desc.block_rows, desc.d_ff), dtype=x.dtype, device=x.device)
    ringattn_ffn_fwd(desc, x, w1, b1, w2, b2, y, workspace, stream=stream)
    return y

