"""ringattn_ring_bwd_noalloc, the ring backward for callers that cannot
allocate: its delta lives in the library's per-GPU scratch array.  Through
the C ABI it must give exactly what ringattn_ring_bwd (delta in a caller
workspace) gives, on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents), and it must refuse a problem
larger than the array before enqueuing anything."""

from __future__ import annotations

import ctypes
import os

import pytest
import torch

from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra

FAKE = 1 << 40  # never dereferenced: the size check comes first


@pytest.mark.skipif(not os.path.exists(ra.LIB_PATH), reason="libringattn.so not built")
def test_noalloc_rejects_problems_beyond_the_scratch():
    d = ra.RaDesc()
    d.batch, d.heads, d.head_dim, d.causal = 1, 64, 128, 1
    d.q_len, d.kv_len, d.q_pos0 = ra.NOALLOC_MAX_ROWS // 64 + 64, 256, 0
    d.in_dtype = d.out_dtype = ra.RA_BF16
    hd = d.heads * d.head_dim
    for arr in (d.q_stride, d.kv_stride, d.o_stride):
        arr[0], arr[1], arr[2] = d.q_len * hd, hd, d.head_dim
    P = ctypes.c_void_p
    one = (P * 1)(FAKE)
    pos = (ctypes.c_int64 * 1)(0)
    st = ra.lib().ringattn_ring_bwd_noalloc(ctypes.byref(d), FAKE, one, one, pos, None, 1, FAKE, FAKE, FAKE, FAKE,
                                            one, one, None)
    assert st == ra.RA_E_UNSUPPORTED
    assert b"scratch" in ra.lib().ringattn_last_error()


def _case(heads, q_len, kv_len, p, q_idx, seed):
    wl = inputs.Workload(f"noalloc H{heads} Q{q_len} P{p}x{kv_len}", "bf16", heads, 128, q_len, kv_len, p, True, q_idx)
    dev = torch.device("cuda:0")
    x = inputs.make_inputs(wl, dev, seed=seed)
    do = inputs.make_grad(wl, dev, seed=seed + 1)
    order = ra.ringattn_ring_order(q_idx, p)
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o, lse = ra.ring_forward(x.q, kb, vb, pos, q_pos0=wl.q_pos0, causal=True)
    return wl, x, do, kb, vb, pos, o, lse


@pytest.mark.gpu
def test_noalloc_equals_ring_bwd_on_two_calls():
    # the second call is smaller: 1 head x 130 rows after 2 heads x 300 rows
    for args in ((2, 300, 200, 4, 2, 120), (1, 130, 128, 3, 1, 130)):
        wl, x, do, kb, vb, pos, o, lse = _case(*args)
        print(f"no-alloc backward: {wl.name}", flush=True)
        dq0, dk0, dv0 = ra.ring_backward(x.q, kb, vb, pos, o, do, lse, q_pos0=wl.q_pos0, causal=True)
        desc = ra.make_desc(x.q, kb[0], o, q_pos0=wl.q_pos0, causal=True)
        dq = torch.full_like(dq0, float("nan"))  # overwritten, like ring_bwd's dq
        dk = [torch.zeros_like(t) for t in dk0]
        dv = [torch.zeros_like(t) for t in dv0]
        ra.ringattn_ring_bwd_noalloc(desc, x.q, kb, vb, pos, o, do, lse, dq, dk, dv)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq0)
        assert all(torch.equal(a, b) for a, b in zip(dk, dk0))
        assert all(torch.equal(a, b) for a, b in zip(dv, dv0))
