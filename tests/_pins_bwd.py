"""Checks that pin the fp64 backward oracle to facts other than itself.

Each takes the oracle backward module (``bwd``) and the forward oracle
(``fwd``, pinned on its own by tests/_pins.py) so that the same checks can run
against copies of the backward with a planted mistake.
"""

from __future__ import annotations

import numpy as np
import torch


def _case(seed, causal=True):
    """Tiny case: 2 heads, 4 query rows at positions 5..8, blocks given out of
    position order with 3, 2 and 4 keys (positions 6.., 0.., 2..)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 4, 2, 3))
    kb = [rng.standard_normal((1, c, 2, 3)) for c in (3, 2, 4)]
    vb = [rng.standard_normal((1, c, 2, 3)) for c in (3, 2, 4)]
    do = rng.standard_normal((1, 4, 2, 3))
    return q, kb, vb, 5, [6, 0, 2], causal, do


def pin_bwd_finite_differences(bwd, fwd):
    """Central differences of L = sum(O * dO), O from the forward oracle, with
    respect to every element of Q, of every K block and of every V block."""
    for causal in (True, False):
        q, kb, vb, q0, pos, _, do = _case(3, causal)
        dq, dk, dv = bwd.ring_attention_bwd(q, kb, vb, q0, pos, causal, do)

        def loss(q_, kb_, vb_):
            o, _ = fwd.ring_attention(q_, kb_, vb_, q0, pos, causal)
            return float((o * do).sum())

        h = 1e-6

        def num_grad(arr, f):
            g = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = arr[idx]
                arr[idx] = old + h
                up = f()
                arr[idx] = old - h
                dn = f()
                arr[idx] = old
                g[idx] = (up - dn) / (2 * h)
            return g

        assert np.allclose(num_grad(q, lambda: loss(q, kb, vb)), dq, rtol=0, atol=1e-7)
        for j in range(len(kb)):
            assert np.allclose(num_grad(kb[j], lambda: loss(q, kb, vb)), dk[j], rtol=0, atol=1e-7)
            assert np.allclose(num_grad(vb[j], lambda: loss(q, kb, vb)), dv[j], rtol=0, atol=1e-7)


def pin_bwd_torch_autograd(bwd, fwd):
    """torch autograd (fp64) of a plain masked softmax attention over the
    concatenated keys, an independent implementation of the same derivative."""
    q, kb, vb, q0, pos, causal, do = _case(5)
    dq, dk, dv = bwd.ring_attention_bwd(q, kb, vb, q0, pos, causal, do)
    qt = torch.tensor(q, requires_grad=True)
    kts = [torch.tensor(k, requires_grad=True) for k in kb]
    vts = [torch.tensor(v, requires_grad=True) for v in vb]
    kpos = torch.cat([p + torch.arange(k.shape[1]) for p, k in zip(pos, kb)])
    qpos = q0 + torch.arange(q.shape[1])
    mask = kpos[None, :] <= qpos[:, None]
    kcat = torch.cat(kts, dim=1)
    vcat = torch.cat(vts, dim=1)
    s = torch.einsum("bqhd,bkhd->bhqk", qt, kcat) / np.sqrt(q.shape[3])
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("bhqk,bkhd->bqhd", torch.softmax(s, dim=-1), vcat)
    (o * torch.tensor(do)).sum().backward()
    assert np.allclose(qt.grad.numpy(), dq, rtol=0, atol=1e-12)
    for j in range(len(kb)):
        assert np.allclose(kts[j].grad.numpy(), dk[j], rtol=0, atol=1e-12)
        assert np.allclose(vts[j].grad.numpy(), dv[j], rtol=0, atol=1e-12)


def pin_bwd_invariants(bwd, fwd):
    """Closed forms: softmax rows sum to 1, so sum_c dV_c = sum_r dO_r over rows
    that see a key; and shifting every key by one vector leaves a non-causal
    output unchanged, so sum_c dK_c = 0."""
    q, kb, vb, q0, pos, _, do = _case(7, causal=False)
    dq, dk, dv = bwd.ring_attention_bwd(q, kb, vb, q0, pos, False, do)
    assert np.allclose(sum(x.sum(axis=1) for x in dv), do.sum(axis=1), rtol=0, atol=1e-12)
    assert np.allclose(sum(x.sum(axis=1) for x in dk), 0.0, rtol=0, atol=1e-12)
    # causal: rows 5..8 each see at least key 0, so the dV identity holds too
    q, kb, vb, q0, pos, _, do = _case(8, causal=True)
    _, _, dv = bwd.ring_attention_bwd(q, kb, vb, q0, pos, True, do)
    assert np.allclose(sum(x.sum(axis=1) for x in dv), do.sum(axis=1), rtol=0, atol=1e-12)


def pin_bwd_delta(bwd, fwd):
    """delta = rowsum(P * dP) = <dO, O>: check it against the softmax and dP
    formed from the forward oracle's probabilities on the same case."""
    q, kb, vb, q0, pos, causal, do = _case(9)
    o, lse = fwd.ring_attention(q, kb, vb, q0, pos, causal)
    d = bwd.delta(o, do)
    kpos = np.concatenate([p + np.arange(k.shape[1]) for p, k in zip(pos, kb)])
    vis = kpos[None, :] <= (q0 + np.arange(q.shape[1]))[:, None]
    for h in range(q.shape[2]):
        kh = np.concatenate([k[0, :, h] for k in kb])
        vh = np.concatenate([v[0, :, h] for v in vb])
        s = np.where(vis, q[0, :, h] @ kh.T / np.sqrt(q.shape[3]), -np.inf)
        p = np.exp(s - lse[0, h][:, None])
        assert np.allclose((p * (do[0, :, h] @ vh.T)).sum(axis=1), d[0, h], rtol=0, atol=1e-12)


def _autograd_grads(q, kb, vb, q0, pos, causal, do, pos_stride=1):
    """dK, dV of every block from torch autograd (fp64) of a plain masked
    softmax attention over the concatenated keys."""
    qt = torch.tensor(q)
    kts = [torch.tensor(k, requires_grad=True) for k in kb]
    vts = [torch.tensor(v, requires_grad=True) for v in vb]
    kpos = torch.cat([p + pos_stride * torch.arange(k.shape[1]) for p, k in zip(pos, kb)])
    qpos = q0 + pos_stride * torch.arange(q.shape[1])
    mask = (kpos[None, :] <= qpos[:, None]) if causal else torch.ones((q.shape[1], kpos.shape[0]), dtype=torch.bool)
    s = torch.einsum("bqhd,bkhd->bhqk", qt, torch.cat(kts, dim=1)) / np.sqrt(q.shape[3])
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1))  # rows without a visible key: no weight
    o = torch.einsum("bhqk,bkhd->bqhd", p, torch.cat(vts, dim=1))
    (o * torch.tensor(do)).sum().backward()
    return [t.grad.numpy() for t in kts], [t.grad.numpy() for t in vts]


def pin_bwd_key_rows(bwd, fwd):
    """The chosen-keys gradient equals the gradient of those keys from torch
    autograd and from the whole-tensor oracle, whatever the row chunking:
    blocks out of position order, keys asked for in a scrambled order with
    repeats, causal and not, striped positions, and query rows that see no
    key at all."""
    q, kb, vb, q0, pos, _, do = _case(11)
    picks = [(2, 3), (0, 0), (1, 1), (2, 0), (0, 2), (1, 0), (2, 3), (0, 1), (2, 1), (2, 2)]
    for causal, q0_, ps in ((True, q0, 1), (False, q0, 1), (True, 1, 1), (True, 2, 3), (True, -5, 1)):
        gk, gv = _autograd_grads(q, kb, vb, q0_, pos, causal, do, pos_stride=ps)
        _, fk, fv = bwd.ring_attention_bwd(q, kb, vb, q0_, pos, causal, do, pos_stride=ps)
        for chunk in (1, 3, 256):
            dk, dv = bwd.key_rows_bwd(q, do, kb, vb, q0_, pos, causal, picks, pos_stride=ps, chunk=chunk)
            for n, (j, i) in enumerate(picks):
                assert np.allclose(dk[:, n], gk[j][:, i], rtol=0, atol=1e-12), (causal, q0_, ps, chunk, j, i)
                assert np.allclose(dv[:, n], gv[j][:, i], rtol=0, atol=1e-12), (causal, q0_, ps, chunk, j, i)
                assert np.allclose(dk[:, n], fk[j][:, i], rtol=0, atol=1e-12)
                assert np.allclose(dv[:, n], fv[j][:, i], rtol=0, atol=1e-12)


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_invariants, pin_bwd_delta,
                pin_bwd_key_rows]
