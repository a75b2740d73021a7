"""Checks that pin the fp64 oracle to facts other than itself.

Each check takes the oracle module as an argument so that the same check can
run against the real oracle (tests/test_oracle_pins.py) and against copies of
it with a planted mistake (tests/test_oracle_planted.py), where at least one
check must fail.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rand_case(seed, b=1, h=2, sq=5, d=4, cks=(4, 3, 6), q_pos0=7, kv_pos0s=(0, 4, 7), scale_in=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, sq, h, d)) * scale_in
    kb = [rng.standard_normal((b, c, h, d)) * scale_in for c in cks]
    vb = [rng.standard_normal((b, c, h, d)) for c in cks]
    return q, kb, vb, q_pos0, list(kv_pos0s)


def pin_mpmath_bruteforce(orc):
    """50-digit direct evaluation: w_j = exp(s_j) with no max subtraction and no
    blocking, O = sum w v / sum w, LSE = log sum w, over visible keys."""
    import mpmath as mp
    mp.mp.dps = 50
    for causal in (False, True):
        for seed in (0, 1):
            q, kb, vb, qp0, kp0 = _rand_case(seed)
            d = q.shape[3]
            o, lse = orc.ring_attention(q, kb, vb, qp0, kp0, causal)
            sc = mp.mpf(1) / mp.sqrt(d)
            for bi in range(q.shape[0]):
                for h in range(q.shape[2]):
                    for r in range(q.shape[1]):
                        qp = qp0 + r
                        num = [mp.mpf(0)] * d
                        den = mp.mpf(0)
                        for kk, vv, p0 in zip(kb, vb, kp0):
                            for j in range(kk.shape[1]):
                                if causal and p0 + j > qp:
                                    continue
                                s = sc * mp.fsum(mp.mpf(float(q[bi, r, h, t])) * mp.mpf(float(kk[bi, j, h, t]))
                                                 for t in range(d))
                                w = mp.exp(s)
                                den += w
                                for t in range(d):
                                    num[t] += w * mp.mpf(float(vv[bi, j, h, t]))
                        if den == 0:
                            assert np.all(o[bi, r, h] == 0) and lse[bi, h, r] == -np.inf
                            continue
                        for t in range(d):
                            ref = num[t] / den
                            assert abs(o[bi, r, h, t] - float(ref)) <= 1e-13 * max(1.0, abs(float(ref))), \
                                (causal, seed, r, t, o[bi, r, h, t], float(ref))
                        ref_lse = float(mp.log(den))
                        assert abs(lse[bi, h, r] - ref_lse) <= 1e-13 * max(1.0, abs(ref_lse))


def pin_single_visible_key(orc):
    """Causal row at global position 0 sees exactly one key: O = v_0, LSE = s_0."""
    rng = np.random.default_rng(3)
    d = 8
    q = rng.standard_normal((1, 3, 2, d))
    k = rng.standard_normal((1, 4, 2, d))
    v = rng.standard_normal((1, 4, 2, d))
    o, lse = orc.ring_attention(q, [k], [v], 0, [0], True)
    for h in range(2):
        s0 = float(q[0, 0, h] @ k[0, 0, h]) / math.sqrt(d)
        assert np.allclose(o[0, 0, h], v[0, 0, h], rtol=0, atol=1e-15)
        assert abs(lse[0, h, 0] - s0) <= 1e-14


def pin_identical_keys(orc):
    """All keys equal: uniform weights, O = mean of visible V, LSE = s + ln n."""
    rng = np.random.default_rng(4)
    d, n = 16, 9
    q = rng.standard_normal((1, 4, 1, d))
    k1 = np.broadcast_to(rng.standard_normal((1, 1, 1, d)), (1, n, 1, d)).copy()
    v = rng.standard_normal((1, n, 1, d))
    blocks_k = [k1[:, :4], k1[:, 4:]]
    blocks_v = [v[:, :4], v[:, 4:]]
    for causal, qp0 in ((False, 0), (True, 3)):
        o, lse = orc.ring_attention(q, blocks_k, blocks_v, qp0, [0, 4], causal)
        for r in range(4):
            nvis = n if not causal else min(n, qp0 + r + 1)
            s = float(q[0, r, 0] @ k1[0, 0, 0]) / math.sqrt(d)
            assert np.allclose(o[0, r, 0], v[0, :nvis, 0].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[0, 0, r] - (s + math.log(nvis))) <= 1e-13


def pin_lse_merge(orc):
    """Per-block results combine into the full result: LSE = logsumexp_b LSE_b and
    O = sum_b exp(LSE_b - LSE) O_b."""
    for causal in (False, True):
        q, kb, vb, qp0, kp0 = _rand_case(5, sq=6, cks=(5, 7, 4))
        o, lse = orc.ring_attention(q, kb, vb, qp0, kp0, causal)
        parts = [orc.ring_attention(q, [k], [v], qp0, [p], causal) for k, v, p in zip(kb, vb, kp0)]
        lses = np.stack([p[1] for p in parts])           # [nb, B, H, Sq]
        mx = np.max(lses, axis=0)
        merged = mx + np.log(np.sum(np.exp(lses - mx), axis=0))
        assert np.allclose(merged, lse, rtol=0, atol=1e-13)
        w = np.exp(lses - lse[None])                      # [nb, B, H, Sq]
        w = np.nan_to_num(w)
        o_m = sum(np.transpose(w[i], (0, 2, 1))[..., None] * parts[i][0] for i in range(len(parts)))
        assert np.allclose(o_m, o, rtol=0, atol=1e-13)


def pin_permutation(orc):
    """Block arrival order does not change the result."""
    q, kb, vb, qp0, kp0 = _rand_case(6, sq=4, cks=(3, 5, 2, 4), kv_pos0s=(0, 3, 8, 10), q_pos0=9)
    for causal in (False, True):
        o, lse = orc.ring_attention(q, kb, vb, qp0, kp0, causal)
        for perm in ([3, 2, 1, 0], [1, 3, 0, 2]):
            o2, lse2 = orc.ring_attention(q, [kb[i] for i in perm], [vb[i] for i in perm], qp0,
                                          [kp0[i] for i in perm], causal)
            assert np.allclose(o2, o, rtol=0, atol=1e-14) and np.allclose(lse2, lse, rtol=0, atol=1e-14)


def pin_shift_invariance(orc):
    """K -> K + u leaves O unchanged and adds scale*<q,u> to LSE; V -> V + w adds w to O."""
    q, kb, vb, qp0, kp0 = _rand_case(7)
    d = q.shape[3]
    rng = np.random.default_rng(8)
    u = rng.standard_normal(d)
    w = rng.standard_normal(d)
    for causal in (False, True):
        o, lse = orc.ring_attention(q, kb, vb, qp0, kp0, causal)
        o2, lse2 = orc.ring_attention(q, [k + u for k in kb], vb, qp0, kp0, causal)
        fin = np.isfinite(lse)
        shift = np.transpose(q @ u, (0, 2, 1)) / math.sqrt(d)   # [B, H, Sq]
        assert np.allclose(o2, o, rtol=0, atol=1e-12)
        assert np.allclose(lse2[fin], (lse + shift)[fin], rtol=0, atol=1e-12)
        o3, _ = orc.ring_attention(q, kb, [v + w for v in vb], qp0, kp0, causal)
        has = np.transpose(fin, (0, 2, 1))[..., None]
        assert np.allclose(np.where(has, o3, 0), np.where(has, o + w, 0), rtol=0, atol=1e-12)


def pin_sdpa(orc):
    """A library routine: torch's scaled_dot_product_attention in fp64 on CPU, with
    an explicit boolean mask for the causal reading."""
    import torch
    import torch.nn.functional as F
    q, kb, vb, qp0, kp0 = _rand_case(9, h=3, sq=7, d=8, cks=(6, 6, 6), kv_pos0s=(0, 6, 12), q_pos0=9)
    for causal in (False, True):
        o, _ = orc.ring_attention(q, kb, vb, qp0, kp0, causal)
        qt = torch.from_numpy(q).permute(0, 2, 1, 3)
        kt = torch.from_numpy(np.concatenate(kb, axis=1)).permute(0, 2, 1, 3)
        vt = torch.from_numpy(np.concatenate(vb, axis=1)).permute(0, 2, 1, 3)
        mask = None
        if causal:
            qpos = torch.arange(q.shape[1]) + qp0
            kpos = torch.arange(kt.shape[2])
            mask = kpos[None, :] <= qpos[:, None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).permute(0, 2, 1, 3).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-13)


def pin_golden(orc):
    """Hand-derived worked examples stored under tests/golden/."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, :, None, :]
        kb = [np.array(b["k"], dtype=np.float64)[None, :, None, :] for b in c["blocks"]]
        vb = [np.array(b["v"], dtype=np.float64)[None, :, None, :] for b in c["blocks"]]
        kp0 = [b["kv_pos0"] for b in c["blocks"]]
        o, lse = orc.ring_attention(q, kb, vb, c["q_pos0"], kp0, c["causal"])
        exp_o = np.array(c["expected_o"], dtype=np.float64)
        exp_l = np.array([float(x) for x in c["expected_lse"]])
        assert np.allclose(o[0, :, 0, :], exp_o, rtol=0, atol=1e-14), (c["name"], o[0, :, 0, :], exp_o)
        fin = np.isfinite(exp_l)
        assert np.array_equal(np.isfinite(lse[0, 0]), fin), c["name"]
        assert np.allclose(lse[0, 0][fin], exp_l[fin], rtol=0, atol=1e-14), (c["name"], lse[0, 0], exp_l)


def pin_partial_state(orc):
    """The (m, l, acc) triple: after all blocks acc/l is O and m + ln l is LSE; m
    is the largest visible score (checked by brute force); states of two
    disjoint block sets merge by the max-rescale rule into the state of the
    union."""
    q, kb, vb, qp0, kp0 = _rand_case(10, sq=6, cks=(4, 4, 4), kv_pos0s=(0, 4, 8), q_pos0=5)
    d = q.shape[3]
    for causal in (False, True):
        o, lse = orc.ring_attention(q, kb, vb, qp0, kp0, causal)
        m, l, acc = orc.partial_state(q, kb, vb, qp0, kp0, causal)
        fin = l > 0
        on = np.transpose(acc / np.where(fin, l, 1)[..., None], (0, 2, 1, 3))
        assert np.allclose(np.where(np.transpose(fin, (0, 2, 1))[..., None], on, 0), o, rtol=0, atol=1e-13)
        assert np.allclose((m + np.log(np.where(fin, l, 1)))[fin], lse[fin], rtol=0, atol=1e-13)
        # m by brute force over visible scores
        for h in range(q.shape[2]):
            for r in range(q.shape[1]):
                best = -np.inf
                for k, p0 in zip(kb, kp0):
                    for j in range(k.shape[1]):
                        if causal and p0 + j > qp0 + r:
                            continue
                        best = max(best, float(q[0, r, h] @ k[0, j, h]) / math.sqrt(d))
                assert m[0, h, r] == best or abs(m[0, h, r] - best) <= 1e-15
        # two disjoint subsets merge to the full state
        ma, la, aa = orc.partial_state(q, kb[:1], vb[:1], qp0, kp0[:1], causal)
        mb, lb, ab = orc.partial_state(q, kb[1:], vb[1:], qp0, kp0[1:], causal)
        mm = np.maximum(ma, mb)
        with np.errstate(invalid="ignore"):
            fa = np.where(np.isfinite(ma), np.exp(ma - mm), 0.0)
            fb = np.where(np.isfinite(mb), np.exp(mb - mm), 0.0)
        assert np.allclose(fa * la + fb * lb, l, rtol=0, atol=1e-12)
        assert np.allclose(fa[..., None] * aa + fb[..., None] * ab, acc, rtol=0, atol=1e-12)


def pin_striped_is_permuted_contiguous(orc):
    """Striped order (pos_stride P): device i holds tokens i, i+P, ... of the
    sequence and block d holds keys d, d+P, ...  Its causal attention must be
    the rows i, i+P, ... of the attention of the whole sequence in natural
    order (one contiguous chunk and block).  The final state of partial_state
    over every block must give the same output and LSE."""
    p, n, h, d = 4, 5, 2, 3
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, p * n, h, d))
    k = rng.standard_normal((1, p * n, h, d))
    v = rng.standard_normal((1, p * n, h, d))
    o_full, lse_full = orc.ring_attention(q, [k], [v], 0, [0], True)
    for i in range(p):
        qi = q[:, i::p]
        kbs = [k[:, dd::p] for dd in range(p)]
        vbs = [v[:, dd::p] for dd in range(p)]
        o, lse = orc.ring_attention(qi, kbs, vbs, i, list(range(p)), True, pos_stride=p)
        assert np.allclose(o, o_full[:, i::p], rtol=0, atol=1e-12)
        assert np.allclose(lse, lse_full[:, :, i::p], rtol=0, atol=1e-12)
        m, l, acc = orc.partial_state(qi, kbs, vbs, i, list(range(p)), True, pos_stride=p)
        o_st = np.transpose(acc / l[..., None], (0, 2, 1, 3))
        assert np.allclose(o_st, o, rtol=0, atol=1e-12)
        assert np.allclose(m + np.log(l), lse, rtol=0, atol=1e-12)


ALL_PINS = [
    pin_striped_is_permuted_contiguous,
    pin_mpmath_bruteforce,
    pin_single_visible_key,
    pin_identical_keys,
    pin_lse_merge,
    pin_permutation,
    pin_shift_invariance,
    pin_sdpa,
    pin_golden,
    pin_partial_state,
]
