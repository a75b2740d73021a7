"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, its host-only helpers are right, and invalid calls return
their status before any HIP call (fake pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest
import torch

from long_context_exact_blockwise_amd import ringattn as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ra.LIB_PATH), reason="libringattn.so not built")


def header_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ringattn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = ra.lib()
    declared = header_symbols()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(ra.SYMBOLS) == declared


def test_abi_version_and_status_strings():
    L = ra.lib()
    assert L.ringattn_abi_version() == ra.ABI_VERSION == 2
    for st in range(8):
        assert L.ringattn_status_str(st).startswith(b"RA_")


def test_ring_order_definition():
    # device q_idx at step s holds the block of device (q_idx - s) mod P
    for p in (1, 2, 4, 8, 128):
        for q_idx in sorted({0, 1 % p, p // 2, p - 1}):
            assert ra.ringattn_ring_order(q_idx, p) == [(q_idx - s) % p for s in range(p)]
    with pytest.raises(ra.RingAttnError) as e:
        ra.ringattn_ring_order(4, 4)
    assert e.value.status == ra.RA_E_SHAPE


def _desc(**kw):
    d = ra.RaDesc()
    d.batch, d.heads, d.head_dim, d.causal = kw.get("batch", 1), kw.get("heads", 2), kw.get("head_dim", 128), \
        kw.get("causal", 1)
    d.q_len, d.kv_len, d.q_pos0 = kw.get("q_len", 256), kw.get("kv_len", 256), kw.get("q_pos0", 512)
    d.scale = kw.get("scale", 0.0)
    d.in_dtype, d.out_dtype = kw.get("in_dtype", ra.RA_BF16), kw.get("out_dtype", ra.RA_BF16)
    d.flags = kw.get("flags", 0)
    d.pos_stride = kw.get("pos_stride", 1)
    hd = d.heads * d.head_dim
    for arr, s in ((d.q_stride, kw.get("q_stride")), (d.kv_stride, kw.get("kv_stride")),
                   (d.o_stride, kw.get("o_stride"))):
        st = s or (d.q_len * hd, hd, d.head_dim)
        for i in range(3):
            arr[i] = st[i]
    return d


def test_block_class():
    d = _desc(q_len=256, kv_len=256, q_pos0=512)
    assert ra.ringattn_block_class(d, 0) == ra.RA_BLOCK_FULL       # keys 0..255 <= rows 512..
    assert ra.ringattn_block_class(d, 256) == ra.RA_BLOCK_FULL     # last key 511 < first row 512
    assert ra.ringattn_block_class(d, 257) == ra.RA_BLOCK_FULL     # last key 512 = first row (inclusive)
    assert ra.ringattn_block_class(d, 258) == ra.RA_BLOCK_DIAG     # last key 513 is after row 512
    assert ra.ringattn_block_class(d, 512) == ra.RA_BLOCK_DIAG
    assert ra.ringattn_block_class(d, 767) == ra.RA_BLOCK_DIAG     # first key 767 = last row
    assert ra.ringattn_block_class(d, 768) == ra.RA_BLOCK_SKIP
    d.causal = 0
    assert ra.ringattn_block_class(d, 10 ** 9) == ra.RA_BLOCK_FULL
    d.kv_len = 0
    assert ra.ringattn_block_class(d, 0) == ra.RA_BLOCK_SKIP
    assert ra.lib().ringattn_block_class(None, 0) == -1


FAKE = 1 << 20  # aligned, never dereferenced: validation fails before any access


def _ring(d, q=FAKE, o=FAKE, lse=FAKE, kb=(FAKE,), vb=(FAKE,), pos=(0,), on_host=0, stage=None, m=None,
          l=None, acc=None, copy=None, compute=None, valid=None):
    L = ra.lib()
    P = ctypes.c_void_p
    n = len(kb) if kb is not None else len(vb)
    karr = (P * max(n, 1))(*kb) if kb is not None else None
    varr = (P * max(n, 1))(*vb) if vb is not None else None
    parr = (ctypes.c_int64 * max(n, 1))(*pos)
    varr_len = (ctypes.c_int64 * max(n, 1))(*valid) if valid is not None else None
    sk = (P * 2)(*stage) if stage else None
    sv = (P * 2)(*stage) if stage else None
    st = L.ringattn_ring_fwd(ctypes.byref(d) if d is not None else None, q, karr, varr, parr, varr_len, n, on_host,
                             sk, sv, m, l, acc, o, lse, compute, copy)
    return st, L.ringattn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), ra.RA_E_UNSUPPORTED),
    (dict(head_dim=256), ra.RA_E_UNSUPPORTED),
    (dict(batch=0), ra.RA_E_SHAPE),
    (dict(heads=0), ra.RA_E_SHAPE),
    (dict(q_len=-1), ra.RA_E_SHAPE),
    (dict(kv_len=-5), ra.RA_E_SHAPE),
    (dict(causal=2), ra.RA_E_SHAPE),
    (dict(scale=float("nan")), ra.RA_E_SHAPE),
    (dict(in_dtype=ra.RA_F32, out_dtype=ra.RA_BF16), ra.RA_E_DTYPE),
    (dict(in_dtype=7), ra.RA_E_DTYPE),
    (dict(q_stride=(256 * 256, 256, 100)), ra.RA_E_ALIGN),   # 200 bytes: rows not 16-byte aligned
    (dict(kv_stride=(256 * 256, 0, 128)), ra.RA_E_SHAPE),    # zero stride along a dim of size > 1
    (dict(kv_stride=(256 * 256, 1 << 24, 128)), ra.RA_E_UNSUPPORTED),
    (dict(kv_len=1 << 30, kv_stride=(128, 128, 128)), ra.RA_E_UNSUPPORTED),  # keys per block must be < 2^30
    (dict(kv_stride=(256 * 256, 64, 128)), ra.RA_E_SHAPE),   # key rows overlap (stride < head_dim)
    (dict(flags=4), ra.RA_E_UNSUPPORTED),
    (dict(pos_stride=-1), ra.RA_E_SHAPE),
    (dict(o_stride=(256 * 256, 256, 64)), ra.RA_E_SHAPE),            # the two heads of a row of O overlap
    (dict(heads=1, o_stride=(256 * 128, 64, 128)), ra.RA_E_SHAPE),   # consecutive rows of O overlap
    (dict(batch=2, o_stride=(1000, 256, 128)), ra.RA_E_SHAPE),       # batch 1 starts inside batch 0
])
def test_descriptor_rejected_before_enqueue(kw, status):
    st, msg = _ring(_desc(**kw))
    assert st == status, (st, msg)
    assert msg


@pytest.mark.parametrize("o_stride", [(2 * 256 * 128, 128, 256 * 128),   # [B, H, S, D]: heads outer
                                      (256 * 256, 256, 128),             # the default [B, S, H, D]
                                      (256 * 512, 512, 256)])            # padded rows
def test_disjoint_output_layouts_pass_the_overlap_check(o_stride):
    st, msg = _ring(_desc(o_stride=o_stride))
    assert st != ra.RA_E_SHAPE, msg


def test_pointer_checks_before_enqueue():
    d = _desc()
    assert _ring(None)[0] == ra.RA_E_NULL
    assert _ring(d, q=None)[0] == ra.RA_E_NULL
    assert _ring(d, o=FAKE + 8)[0] == ra.RA_E_ALIGN
    assert _ring(d, kb=(FAKE + 4,))[0] == ra.RA_E_ALIGN
    assert _ring(d, kb=None)[0] == ra.RA_E_NULL
    assert _ring(d, on_host=2)[0] == ra.RA_E_SHAPE
    # host-streamed needs staging slots, a workspace, and two streams
    assert _ring(d, on_host=1)[0] == ra.RA_E_NULL
    st, msg = _ring(d, on_host=1, stage=(FAKE, FAKE), m=FAKE, l=FAKE, acc=FAKE)
    assert st == ra.RA_E_SHAPE and "stream" in msg
    d2 = _desc(flags=ra.RA_FLAG_PERBLOCK)
    assert _ring(d2)[0] == ra.RA_E_NULL  # per-block path needs the state workspace
    L = ra.lib()
    assert L.ringattn_block_fwd(ctypes.byref(d), FAKE, None, FAKE, 0, FAKE, FAKE, FAKE, None) == ra.RA_E_NULL
    assert L.ringattn_finalize(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 2, FAKE, None) == ra.RA_E_ALIGN
    assert L.ringattn_init_state(ctypes.byref(d), None, FAKE, FAKE, None) == ra.RA_E_NULL
    assert L.ringattn_probe_copy(FAKE, FAKE, 15, None) == ra.RA_E_SHAPE


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_valid_call_without_device_reports_hip_error():
    st, msg = _ring(_desc())
    assert st in (ra.RA_E_HIP, ra.RA_E_MEMTYPE), (st, msg)
    assert msg


@pytest.mark.parametrize("valid", [(-1,), (257,)])
def test_valid_length_out_of_range_rejected(valid):
    """kv_valid[i] must lie in [0, kv_len]; checked before anything is enqueued."""
    st, msg = _ring(_desc(kv_len=256), valid=valid)
    assert st == ra.RA_E_SHAPE and "kv_valid" in msg, (st, msg)


def _floor_div(a, b):
    return a // b  # Python floors


@pytest.mark.parametrize("p,i", [(4, 0), (4, 3), (8, 5)])
def test_block_class_striped_matches_brute_force(p, i):
    """With pos_stride P (striped order), the class of block d follows from the
    visibility of key j*P + d to row r*P + i, enumerated directly."""
    n = 8
    d = _desc(q_len=n, kv_len=n, q_pos0=i, pos_stride=p, q_stride=(n * 256, 256, 128),
              kv_stride=(n * 256, 256, 128), o_stride=(n * 256, 256, 128))
    for dev in range(p):
        vis = [[j * p + dev <= r * p + i for j in range(n)] for r in range(n)]
        flat = [x for row in vis for x in row]
        want = ra.RA_BLOCK_FULL if all(flat) else (ra.RA_BLOCK_SKIP if not any(flat) else ra.RA_BLOCK_DIAG)
        assert ra.ringattn_block_class(d, dev) == want, (dev, p, i)
    # a block placed far after the chunk (key 0 after the last row) is skipped
    assert ra.ringattn_block_class(d, (n - 1) * p + i + 1) == ra.RA_BLOCK_SKIP
    d.pos_stride = -2
    assert ra.ringattn_block_class(d, 0) == -1



def _ring_bwd(d, kb=(FAKE,), pos=(0,), valid=None, n=None, dk=(FAKE,), q=FAKE):
    L = ra.lib()
    P = ctypes.c_void_p
    n = len(kb) if n is None else n
    arr = lambda xs: (P * max(len(xs), 1))(*xs) if xs is not None else None  # noqa: E731
    parr = (ctypes.c_int64 * max(len(pos), 1))(*pos)
    varr = (ctypes.c_int64 * max(len(pos), 1))(*valid) if valid is not None else None
    st = L.ringattn_ring_bwd(ctypes.byref(d), q, arr(kb), arr(kb), parr, varr, n, FAKE, FAKE, FAKE, FAKE, FAKE,
                             arr(dk), arr(dk), None)
    return st, L.ringattn_last_error().decode()


def test_backward_checks_before_enqueue():
    """The backward entry points validate like the forward and take bf16
    inputs only."""
    L = ra.lib()
    st, msg = _ring_bwd(_desc(in_dtype=ra.RA_F32, out_dtype=ra.RA_F32))
    assert st == ra.RA_E_UNSUPPORTED and "bf16" in msg, (st, msg)
    assert _ring_bwd(_desc(head_dim=96))[0] == ra.RA_E_UNSUPPORTED
    assert _ring_bwd(_desc(), n=-1)[0] == ra.RA_E_SHAPE
    assert _ring_bwd(_desc(), q=None)[0] == ra.RA_E_NULL
    assert _ring_bwd(_desc(), dk=None)[0] == ra.RA_E_NULL
    assert _ring_bwd(_desc(), dk=(FAKE + 4,))[0] == ra.RA_E_ALIGN
    st, msg = _ring_bwd(_desc(kv_len=256), valid=(300,))
    assert st == ra.RA_E_SHAPE and "kv_valid" in msg
    d = _desc()
    assert L.ringattn_block_bwd(ctypes.byref(d), FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None) == ra.RA_E_NULL
    assert L.ringattn_bwd_delta(ctypes.byref(d), FAKE, FAKE, FAKE + 2, None) == ra.RA_E_ALIGN
    d32 = _desc(in_dtype=ra.RA_F32, out_dtype=ra.RA_F32)
    assert L.ringattn_bwd_delta(ctypes.byref(d32), FAKE, FAKE, FAKE, None) == ra.RA_E_UNSUPPORTED


def _ffn(**kw):
    d = ra.RaFfnDesc()
    d.rows, d.d_model, d.d_ff = kw.get("rows", 256), kw.get("d_model", 128), kw.get("d_ff", 512)
    d.x_stride, d.y_stride = kw.get("x_stride", d.d_model), kw.get("y_stride", d.d_model)
    d.block_rows = kw.get("block_rows", 128)
    ptrs = kw.get("ptrs", [FAKE] * 7)
    st = ra.lib().ringattn_ffn_fwd(ctypes.byref(d), *ptrs, None)
    return st, ra.lib().ringattn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), ra.RA_E_SHAPE),
    (dict(d_model=0), ra.RA_E_SHAPE),
    (dict(d_model=96), ra.RA_E_UNSUPPORTED),
    (dict(d_ff=100), ra.RA_E_UNSUPPORTED),
    (dict(d_ff=1 << 17), ra.RA_E_UNSUPPORTED),
    (dict(x_stride=64), ra.RA_E_SHAPE),
    (dict(y_stride=132), ra.RA_E_ALIGN),
    (dict(x_stride=1 << 22), ra.RA_E_UNSUPPORTED),
    (dict(block_rows=0), ra.RA_E_SHAPE),
    (dict(ptrs=[FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE]), ra.RA_E_NULL),
    (dict(ptrs=[FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE]), ra.RA_E_ALIGN),
])
def test_ffn_checks_before_enqueue(kw, status):
    st, msg = _ffn(**kw)
    assert st == status, (st, msg)
    assert msg


def test_ffn_empty_chunk_needs_no_pointers():
    assert _ffn(rows=0, ptrs=[None] * 7)[0] == ra.RA_OK


def test_probe_mfma_checks_before_enqueue():
    L = ra.lib()
    assert L.ringattn_probe_mfma(None, 1, 1, None) == ra.RA_E_NULL
    assert L.ringattn_probe_mfma(FAKE + 4, 1, 1, None) == ra.RA_E_ALIGN
    assert L.ringattn_probe_mfma(FAKE, 0, 1, None) == ra.RA_E_SHAPE
    assert L.ringattn_probe_mfma(FAKE, 1, 0, None) == ra.RA_E_SHAPE


def test_probe_mfma_data_checks_before_enqueue():
    L = ra.lib()
    assert L.ringattn_probe_mfma_data(None, FAKE, 1, 1, None) == ra.RA_E_NULL
    assert L.ringattn_probe_mfma_data(FAKE, None, 1, 1, None) == ra.RA_E_NULL
    assert L.ringattn_probe_mfma_data(FAKE + 8, FAKE, 1, 1, None) == ra.RA_E_ALIGN
    assert L.ringattn_probe_mfma_data(FAKE, FAKE, 0, 1, None) == ra.RA_E_SHAPE
    assert L.ringattn_probe_mfma_data(FAKE, FAKE, 1, 1 << 25, None) == ra.RA_E_SHAPE


def test_probe_mfma_lds_checks_before_enqueue():
    L = ra.lib()
    assert L.ringattn_probe_mfma_lds(None, FAKE, 1, 1, 16, None) == ra.RA_E_NULL
    assert L.ringattn_probe_mfma_lds(FAKE, None, 1, 1, 16, None) == ra.RA_E_NULL
    assert L.ringattn_probe_mfma_lds(FAKE + 8, FAKE, 1, 1, 16, None) == ra.RA_E_ALIGN
    assert L.ringattn_probe_mfma_lds(FAKE, FAKE, 0, 1, 16, None) == ra.RA_E_SHAPE
    assert L.ringattn_probe_mfma_lds(FAKE, FAKE, 1, 1 << 23, 16, None) == ra.RA_E_SHAPE
    for bad in (0, 2, 12, 32, -16):
        assert L.ringattn_probe_mfma_lds(FAKE, FAKE, 1, 1, bad, None) == ra.RA_E_SHAPE
