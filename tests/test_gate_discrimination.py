"""The fp32 gate (max-abs 1e-5) must tell the exact online-softmax merge from the
per-chunk merge printed in the PyTorch section of "Ring Attention: Train 1M
Tokens on 8GB GPUs in 2026", which weights
each chunk's softmax output by that chunk's exp-sum taken against the chunk's
own maximum and never brings the chunks to a common maximum."""

import numpy as np

import oracle
from long_context_exact_blockwise_amd import inputs


def _page_merge(q, kb, vb, scale):
    """The page's per-chunk rule, restated: out += softmax_b(S) V * expsum_b,
    den += expsum_b, result out/den, with expsum_b = sum exp(S - max_b S)."""
    out = 0.0
    den = 0.0
    for k, v in zip(kb, vb):
        s = scale * (q @ k.T)
        mb = s.max(axis=1, keepdims=True)
        e = np.exp(s - mb)
        es = e.sum(axis=1, keepdims=True)
        out = out + (e / es) @ v * es
        den = den + es
    return out / den


def _online_merge(q, kb, vb, scale):
    """The exact rule: common running max, rescale of the carried sum and output."""
    n = q.shape[0]
    m = np.full((n, 1), -np.inf)
    l = np.zeros((n, 1))
    acc = np.zeros((n, vb[0].shape[1]))
    for k, v in zip(kb, vb):
        s = scale * (q @ k.T)
        m_new = np.maximum(m, s.max(axis=1, keepdims=True))
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new)
        l = alpha * l + p.sum(axis=1, keepdims=True)
        acc = alpha * acc + p @ v
        m = m_new
    return acc / l


def test_page_merge_fails_fp32_gate_exact_merge_passes():
    wl = inputs.CONFIGS[1]
    x = inputs.make_inputs(wl, "cpu", seed=0)
    q = inputs.to_f64(x.q)[0, :, 0, :]
    kb = [inputs.to_f64(x.k_block(j))[0, :, 0, :] for j in range(wl.num_blocks)]
    vb = [inputs.to_f64(x.v_block(j))[0, :, 0, :] for j in range(wl.num_blocks)]
    ref, _ = oracle.ring_attention(inputs.to_f64(x.q), [b[None, :, None, :] for b in kb],
                                   [b[None, :, None, :] for b in vb], wl.q_pos0,
                                   [wl.kv_pos0(j) for j in range(wl.num_blocks)], wl.causal)
    ref = ref[0, :, 0, :]
    scale = 1.0 / np.sqrt(wl.head_dim)
    err_page = np.abs(_page_merge(q, kb, vb, scale) - ref).max()
    err_exact = np.abs(_online_merge(q, kb, vb, scale) - ref).max()
    assert err_page > 1e-3, err_page
    assert err_exact < 1e-12, err_exact
