"""GPU parity of the backward pass (dQ of the local chunk, this chunk's dK and
dV contribution for every block of the ring) against the fp64 backward oracle.

Tolerance (bf16 inputs, fp32 results).  Every product the kernels form has one
or two bf16-rounded operands (Q, K, V, dO exactly as given; P and dS rounded
from fp32, relative error <= 2^-9 each), so each term of a gradient sum carries
a relative error of at most about 2^-8, and delta = <dO, O> uses the forward's
bf16 O.  Summed with independent signs, the error of a whole gradient tensor
stays near that per-term size (2^-8 = 3.9e-3): the tests hold the relative
Frobenius error of each tensor to 5e-3 and every element to 1e-2 of the
tensor's largest magnitude (entries of a gradient sum can cancel, so an element-relative bound
is not meaningful).  Padding past a block's valid length must get no gradient
and must not be read.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra
from tests._gpu_common import cuda, small

pytestmark = pytest.mark.gpu

FRO_TOL = 5e-3
MAX_TOL = 1e-2


def _check(gpu, ref, what):
    g = gpu.detach().double().cpu().numpy() if torch.is_tensor(gpu) else gpu
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    nref = float(np.linalg.norm(ref))
    err = g - ref
    if nref == 0.0:
        assert not np.any(g), f"{what}: gradient expected to be exactly zero"
        return {"what": what, "zero": True}
    fro = float(np.linalg.norm(err)) / nref
    mx = float(np.max(np.abs(err))) / float(np.max(np.abs(ref)))
    assert fro <= FRO_TOL, f"{what}: relative Frobenius error {fro:.3e} > {FRO_TOL}"
    assert mx <= MAX_TOL, f"{what}: max error / max|ref| {mx:.3e} > {MAX_TOL}"
    return {"what": what, "fro": fro, "max_scaled": mx}


def _oracle_bwd(x, do, q_pos0, kv_pos0s, causal, valid=None, pos_stride=1, blocks=None):
    """Oracle gradients, one head at a time; blocks: the block indices in the
    order passed (their dK/dV come back in that order)."""
    wl = x.wl
    blocks = list(range(wl.num_blocks)) if blocks is None else list(blocks)
    valid = [wl.kv_len] * wl.num_blocks if valid is None else valid
    dq, dk, dv = [], [[] for _ in blocks], [[] for _ in blocks]
    for h in range(wl.heads):
        q = inputs.to_f64(x.q[:, :, h:h + 1, :])
        g = inputs.to_f64(do[:, :, h:h + 1, :])
        kb = [inputs.to_f64(x.k_block(j)[:, :valid[j], h:h + 1, :]) for j in blocks]
        vb = [inputs.to_f64(x.v_block(j)[:, :valid[j], h:h + 1, :]) for j in blocks]
        a, b, c = oracle.ring_attention_bwd(q, kb, vb, q_pos0, [kv_pos0s[j] for j in blocks], causal, g,
                                            pos_stride=pos_stride)
        dq.append(a)
        for i in range(len(blocks)):
            dk[i].append(b[i])
            dv[i].append(c[i])
    return (np.concatenate(dq, axis=2), [np.concatenate(t, axis=2) for t in dk],
            [np.concatenate(t, axis=2) for t in dv])


def _run(x, do, order, kv_pos0s, q_pos0, causal, valid=None, pos_stride=1):
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    pos = [kv_pos0s[j] for j in order]
    vo = None if valid is None else [valid[j] for j in order]
    o, lse = ra.ring_forward(x.q, kb, vb, pos, q_pos0=q_pos0, causal=causal, kv_valid=vo, pos_stride=pos_stride)
    dq, dk, dv = ra.ring_backward(x.q, kb, vb, pos, o, do, lse, q_pos0=q_pos0, causal=causal, kv_valid=vo,
                                  pos_stride=pos_stride)
    torch.cuda.synchronize()
    return dq, dk, dv


def _poison_padding(x, valid):
    for j, n in enumerate(valid):
        x.k_block(j)[:, n:] = float("nan")
        x.v_block(j)[:, n:] = float("nan")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("q_idx", [2, 0])
def test_ring_backward_matches_oracle(d, causal, q_idx):
    """300 query rows (two full 128-row tiles and a ragged one), four blocks of
    200 keys (three full 64-key tiles and a ragged one), in ring order."""
    wl = small(d=d, q_len=300, kv_len=200, p=4, causal=causal, q_idx=q_idx)
    x = inputs.make_inputs(wl, cuda(), seed=50 + d + q_idx)
    do = inputs.make_grad(wl, cuda(), seed=60 + d)
    order = ra.ringattn_ring_order(q_idx, wl.num_blocks)
    kv_pos0s = [wl.kv_pos0(j) for j in range(wl.num_blocks)]
    dq, dk, dv = _run(x, do, order, kv_pos0s, wl.q_pos0, causal)
    rq, rk, rv = _oracle_bwd(x, do, wl.q_pos0, kv_pos0s, causal, blocks=order)
    out = [_check(dq, rq, "dQ")]
    for i, j in enumerate(order):
        out.append(_check(dk[i], rk[i], f"dK block {j}"))
        out.append(_check(dv[i], rv[i], f"dV block {j}"))
    print(out)


def test_valid_lengths_backward():
    """Blocks of unequal length (full, empty, ragged, one tile) with NaN in
    the padding: gradients match the oracle on the truncated blocks and the
    padding rows of dK, dV stay zero."""
    valid = [200, 0, 137, 64]
    wl = small(q_len=300, kv_len=200, p=4, causal=True, q_idx=2)
    x = inputs.make_inputs(wl, cuda(), seed=70)
    do = inputs.make_grad(wl, cuda(), seed=71)
    _poison_padding(x, valid)
    order = ra.ringattn_ring_order(2, 4)
    kv_pos0s = [wl.kv_pos0(j) for j in range(4)]
    dq, dk, dv = _run(x, do, order, kv_pos0s, wl.q_pos0, True, valid=valid)
    rq, rk, rv = _oracle_bwd(x, do, wl.q_pos0, kv_pos0s, True, valid=valid, blocks=order)
    out = [_check(dq, rq, "dQ")]
    for i, j in enumerate(order):
        n = valid[j]
        assert torch.count_nonzero(dk[i][:, n:]) == 0 and torch.count_nonzero(dv[i][:, n:]) == 0
        out.append(_check(dk[i][:, :n], rk[i], f"dK block {j}"))
        out.append(_check(dv[i][:, :n], rv[i], f"dV block {j}"))
    print(out)


@pytest.mark.parametrize("dev", [0, 3])
def test_striped_backward(dev):
    p, n = 4, 200
    wl = small(q_len=n, kv_len=n, p=p, q_idx=dev)
    x = inputs.make_inputs(wl, cuda(), seed=80 + dev)
    do = inputs.make_grad(wl, cuda(), seed=90 + dev)
    order = ra.ringattn_ring_order(dev, p)
    dq, dk, dv = _run(x, do, order, list(range(p)), dev, True, pos_stride=p)
    rq, rk, rv = _oracle_bwd(x, do, dev, list(range(p)), True, pos_stride=p, blocks=order)
    out = [_check(dq, rq, "dQ")]
    for i, j in enumerate(order):
        out.append(_check(dk[i], rk[i], f"dK block {j}"))
        out.append(_check(dv[i], rv[i], f"dV block {j}"))
    print(out)


def test_rows_without_keys_get_no_gradient():
    """Every block empty: every LSE is -inf and every gradient exactly zero."""
    wl = small(q_len=130, kv_len=128, p=3, q_idx=2)
    x = inputs.make_inputs(wl, cuda(), seed=72)
    do = inputs.make_grad(wl, cuda(), seed=73)
    _poison_padding(x, [0, 0, 0])
    dq, dk, dv = _run(x, do, [0, 1, 2], [wl.kv_pos0(j) for j in range(3)], wl.q_pos0, True, valid=[0, 0, 0])
    assert torch.count_nonzero(dq) == 0
    assert all(torch.count_nonzero(t) == 0 for t in dk + dv)


def test_ring_bwd_accumulates_into_dk_dv():
    """dK, dV are added to what the buffers hold; dQ is overwritten."""
    wl = small(q_len=200, kv_len=160, p=2, q_idx=1)
    x = inputs.make_inputs(wl, cuda(), seed=74)
    do = inputs.make_grad(wl, cuda(), seed=75)
    kb = [x.k_block(j) for j in (1, 0)]
    vb = [x.v_block(j) for j in (1, 0)]
    pos = [wl.kv_pos0(j) for j in (1, 0)]
    o, lse = ra.ring_forward(x.q, kb, vb, pos, q_pos0=wl.q_pos0, causal=True)
    dq0, dk0, dv0 = ra.ring_backward(x.q, kb, vb, pos, o, do, lse, q_pos0=wl.q_pos0, causal=True)
    desc = ra.make_desc(x.q, kb[0], o, q_pos0=wl.q_pos0, causal=True)
    delta = torch.empty((1, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
    dq = torch.full_like(dq0, 7.0)
    dk = [torch.full_like(t, 1.5) for t in dk0]
    dv = [torch.full_like(t, -2.0) for t in dv0]
    ra.ringattn_ring_bwd(desc, x.q, kb, vb, pos, o, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0)
    for a, b in zip(dk, dk0):
        assert torch.allclose(a - 1.5, b, rtol=0, atol=1e-6)
    for a, b in zip(dv, dv0):
        assert torch.allclose(a + 2.0, b, rtol=0, atol=1e-6)


def test_block_bwd_steps_equal_ring_bwd():
    """delta, zeroed dQ and one block_bwd call per block reproduce ring_bwd."""
    wl = small(q_len=260, kv_len=192, p=3, q_idx=2, d=64)
    x = inputs.make_inputs(wl, cuda(), seed=76)
    do = inputs.make_grad(wl, cuda(), seed=77)
    order = ra.ringattn_ring_order(2, 3)
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o, lse = ra.ring_forward(x.q, kb, vb, pos, q_pos0=wl.q_pos0, causal=True)
    dq0, dk0, dv0 = ra.ring_backward(x.q, kb, vb, pos, o, do, lse, q_pos0=wl.q_pos0, causal=True)
    desc = ra.make_desc(x.q, kb[0], o, q_pos0=wl.q_pos0, causal=True)
    delta = torch.empty((1, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
    ra.ringattn_bwd_delta(desc, o, do, delta)
    dq = torch.zeros_like(dq0)
    dk = [torch.zeros_like(t) for t in dk0]
    dv = [torch.zeros_like(t) for t in dv0]
    for i in range(3):
        ra.ringattn_block_bwd(desc, x.q, kb[i], vb[i], pos[i], do, lse, delta, dq, dk[i], dv[i])
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0)
    assert all(torch.equal(a, b) for a, b in zip(dk, dk0))
    assert all(torch.equal(a, b) for a, b in zip(dv, dv0))
    ref = (o.float() * do.float()).sum(dim=3).permute(0, 2, 1)
    assert torch.allclose(delta, ref, rtol=1e-5, atol=1e-5)


def test_medium_backward_matches_oracle():
    """2048 query rows against four blocks of 2048 keys, causal, last device:
    many key and query tiles per workgroup."""
    wl = small(heads=1, q_len=2048, kv_len=2048, p=4, causal=True, q_idx=3)
    x = inputs.make_inputs(wl, cuda(), seed=78)
    do = inputs.make_grad(wl, cuda(), seed=79)
    order = ra.ringattn_ring_order(3, 4)
    kv_pos0s = [wl.kv_pos0(j) for j in range(4)]
    dq, dk, dv = _run(x, do, order, kv_pos0s, wl.q_pos0, True)
    rq, rk, rv = _oracle_bwd(x, do, wl.q_pos0, kv_pos0s, True, blocks=order)
    out = [_check(dq, rq, "dQ")]
    for i, j in enumerate(order):
        out.append(_check(dk[i], rk[i], f"dK block {j}"))
        out.append(_check(dv[i], rv[i], f"dV block {j}"))
    print(out)


def test_full_size_backward_sampled():
    """32768 query rows against 8 blocks of 32768 keys, 16 heads, causal, last
    device of the ring, in the launch configuration the benchmark times: dQ of
    two windows of rows of two heads against the oracle; for every head,
    sum_c dK_c = 0 (a common shift of all keys leaves every softmax row
    unchanged) and sum_c dV_c = sum_r dO_r (every row sees a key and its
    softmax row sums to 1), in fp64 over the fp32 results."""
    wl = inputs.CONFIGS[2]
    print(f"config 2: {wl.name}", flush=True)
    x = inputs.make_inputs(wl, cuda(), seed=0)
    do = inputs.make_grad(wl, cuda(), seed=1)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    kv_pos0s = [wl.kv_pos0(j) for j in range(wl.num_blocks)]
    dq, dk, dv = _run(x, do, order, kv_pos0s, wl.q_pos0, True)
    assert torch.isfinite(dq).all() and all(torch.isfinite(t).all() for t in dk + dv)
    for h in (0, wl.heads - 1):
        kbh = [inputs.to_f64(x.k_block(j)[:, :, h:h + 1, :]) for j in range(wl.num_blocks)]
        vbh = [inputs.to_f64(x.v_block(j)[:, :, h:h + 1, :]) for j in range(wl.num_blocks)]
        for a, b in ((0, 4), (wl.q_len - 8, wl.q_len)):
            q = inputs.to_f64(x.q[:, a:b, h:h + 1, :])
            g = inputs.to_f64(do[:, a:b, h:h + 1, :])
            rq, _, _ = oracle.ring_attention_bwd(q, kbh, vbh, wl.q_pos0 + a, kv_pos0s, True, g)
            print(_check(dq[:, a:b, h:h + 1, :], rq, f"dQ rows {a}..{b - 1} head {h}"))
    for h in range(wl.heads):
        sdk = sum(t[:, :, h].double().sum(dim=1) for t in dk)
        mk = sum(t[:, :, h].double().abs().sum(dim=1) for t in dk).max()
        sdv = sum(t[:, :, h].double().sum(dim=1) for t in dv)
        mv = sum(t[:, :, h].double().abs().sum(dim=1) for t in dv).max()
        sdo = do[:, :, h].double().sum(dim=1)
        ek = float(sdk.abs().max() / mk)
        ev = float((sdv - sdo).abs().max() / mv)
        assert ek <= 1e-3 and ev <= 1e-3, (h, ek, ev)


@pytest.mark.parametrize("d", [128, 64])
def test_striped_with_valid_lengths_backward(d):
    """Both extensions at once: striped positions (P = 4) and blocks of
    unequal length with NaN in the padding."""
    p, n = 4, 160
    valid = [160, 97, 0, 64]
    wl = small(d=d, q_len=n, kv_len=n, p=p, q_idx=2)
    x = inputs.make_inputs(wl, cuda(), seed=110 + d)
    do = inputs.make_grad(wl, cuda(), seed=111 + d)
    _poison_padding(x, valid)
    order = ra.ringattn_ring_order(2, p)
    dq, dk, dv = _run(x, do, order, list(range(p)), 2, True, valid=valid, pos_stride=p)
    rq, rk, rv = _oracle_bwd(x, do, 2, list(range(p)), True, valid=valid, pos_stride=p, blocks=order)
    out = [_check(dq, rq, "dQ")]
    for i, j in enumerate(order):
        m = valid[j]
        assert torch.count_nonzero(dk[i][:, m:]) == 0 and torch.count_nonzero(dv[i][:, m:]) == 0
        out.append(_check(dk[i][:, :m], rk[i], f"dK block {j}"))
        out.append(_check(dv[i][:, :m], rv[i], f"dV block {j}"))
    print(out)
