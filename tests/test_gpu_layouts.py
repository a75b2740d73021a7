"""GPU parity for batch > 1 and for strided (non-dense) layouts: Q, K, V as
views of one packed [B, S, 3, H, D] tensor, forward and backward, against
the fp64 oracles."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra
from tests._gpu_common import compare, cuda, gpu_rows

pytestmark = pytest.mark.gpu


def _wl(batch, causal=True, d=128, q_len=200, kv_len=136, p=3, q_idx=2):
    return inputs.Workload(f"layout B{batch} D{d}", "bf16", 2, d, q_len, kv_len, p, causal, q_idx, batch=batch)


def _oracle_fwd(q, kb, vb, q_pos0, pos, causal):
    f = inputs.to_f64
    return oracle.ring_attention(f(q), [f(k) for k in kb], [f(v) for v in vb], q_pos0, pos, causal)


@pytest.mark.parametrize("perblock", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_batch_two_forward(perblock, d):
    wl = _wl(2, d=d)
    x = inputs.make_inputs(wl, cuda(), seed=90 + d)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o, lse = ra.ring_forward(x.q, kb, vb, pos, q_pos0=wl.q_pos0, causal=True, perblock=perblock)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle_fwd(x.q, kb, vb, wl.q_pos0, pos, True)
    print(compare(*gpu_rows(o, lse), ref_o, ref_l, "bf16", f"batch 2 D{d} perblock={perblock}"))


def _packed(wl, seed):
    """Q, K, V of the workload as strided views of one [B, S, 3, H, D] bf16
    tensor (S = P*Ck; the query chunk is the first q_len rows of its own
    packed buffer)."""
    x = inputs.make_inputs(wl, cuda(), seed=seed)
    b, h, d = wl.batch, wl.heads, wl.head_dim
    n = wl.num_blocks * wl.kv_len
    kv = torch.empty((b, n, 3, h, d), dtype=torch.bfloat16, device=x.q.device)
    kv[:, :, 1] = x.k
    kv[:, :, 2] = x.v
    qbuf = torch.empty((b, wl.q_len, 3, h, d), dtype=torch.bfloat16, device=x.q.device)
    qbuf[:, :, 0] = x.q
    k = kv[:, :, 1]
    v = kv[:, :, 2]
    q = qbuf[:, :, 0]
    assert q.stride() == (wl.q_len * 3 * h * d, 3 * h * d, d, 1) and not q.is_contiguous()
    return x, q, k, v, qbuf


@pytest.mark.parametrize("perblock", [False, True])
def test_packed_qkv_forward(perblock):
    wl = _wl(2)
    x, q, k, v, _ = _packed(wl, 95)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    kb = [k[:, j * wl.kv_len:(j + 1) * wl.kv_len] for j in order]
    vb = [v[:, j * wl.kv_len:(j + 1) * wl.kv_len] for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o, lse = ra.ring_forward(q, kb, vb, pos, q_pos0=wl.q_pos0, causal=True, perblock=perblock)
    o_ref, lse_ref = ra.ring_forward(x.q, [x.k_block(j) for j in order], [x.v_block(j) for j in order], pos,
                                     q_pos0=wl.q_pos0, causal=True, perblock=perblock)
    torch.cuda.synchronize()
    # the same arithmetic on the same values: identical to the dense layout
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    ref_o, ref_l = _oracle_fwd(x.q, [x.k_block(j) for j in order], [x.v_block(j) for j in order],
                               wl.q_pos0, pos, True)
    print(compare(*gpu_rows(o, lse), ref_o, ref_l, "bf16", "packed qkv"))


def _bwd_check(g, ref, what):
    g = g.detach().double().cpu().numpy()
    nref = float(np.linalg.norm(ref))
    if nref == 0.0:
        assert not np.any(g), what
        return
    fro = float(np.linalg.norm(g - ref)) / nref
    mx = float(np.max(np.abs(g - ref))) / float(np.max(np.abs(ref)))
    assert fro <= 5e-3 and mx <= 1e-2, (what, fro, mx)


@pytest.mark.parametrize("packed", [False, True])
def test_batch_two_backward(packed):
    """Gradients for batch 2, with dense or packed-QKV inputs (dO then has
    the packed query layout too)."""
    wl = _wl(2)
    if packed:
        x, q, k, v, _ = _packed(wl, 97)
    else:
        x = inputs.make_inputs(wl, cuda(), seed=97)
        q, k, v = x.q, x.k, x.v
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    kb = [k[:, j * wl.kv_len:(j + 1) * wl.kv_len] for j in order]
    vb = [v[:, j * wl.kv_len:(j + 1) * wl.kv_len] for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o, lse = ra.ring_forward(q, kb, vb, pos, q_pos0=wl.q_pos0, causal=True)
    do_dense = inputs.make_grad(wl, cuda(), seed=98)
    if packed:
        dbuf = torch.zeros((wl.batch, wl.q_len, 3, wl.heads, wl.head_dim), dtype=torch.bfloat16, device=q.device)
        dbuf[:, :, 0] = do_dense
        do = dbuf[:, :, 0]
    else:
        do = do_dense
    dq, dk, dv = ra.ring_backward(q, kb, vb, pos, o, do, lse, q_pos0=wl.q_pos0, causal=True)
    torch.cuda.synchronize()
    f = inputs.to_f64
    rq, rk, rv = oracle.ring_attention_bwd(f(x.q), [f(x.k_block(j)) for j in order], [f(x.v_block(j)) for j in order],
                                           wl.q_pos0, pos, True, f(do_dense))
    _bwd_check(dq, rq, "dQ")
    for i in range(len(order)):
        _bwd_check(dk[i], rk[i], f"dK {i}")
        _bwd_check(dv[i], rv[i], f"dV {i}")
