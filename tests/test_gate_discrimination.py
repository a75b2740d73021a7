"""The fp32 gate (max-abs 1e-5) must tell the exact online-softmax merge from
the per-chunk merge of the PyTorch section of "Ring Attention: Train 1M Tokens
on 8GB GPUs in 2026" ("Building Ring Attention in PyTorch"), which adds up
each chunk's exp-weighted output and exp-sum, each taken against that chunk's
own maximum, and never brings the chunks to a common maximum.

Both merges are written here from the per-block state (m_b, l_b, acc_b) of
each block on its own, the closed form ``oracle.partial_state`` gives:
  wrong: O = sum_b acc_b / sum_b l_b              (no common maximum)
  exact: O = sum_b e^(m_b - M) acc_b / sum_b e^(m_b - M) l_b,  M = max_b m_b
"""

import numpy as np

import oracle
from long_context_exact_blockwise_amd import inputs


def _block_states(x, wl):
    q = inputs.to_f64(x.q)
    states = []
    for j in range(wl.num_blocks):
        m, l, acc = oracle.partial_state(q, [inputs.to_f64(x.k_block(j))], [inputs.to_f64(x.v_block(j))], wl.q_pos0,
                                         [wl.kv_pos0(j)], wl.causal)
        states.append((m[0, 0], l[0, 0], acc[0, 0]))
    return states


def _merge_without_common_max(states):
    acc = sum(s[2] for s in states)
    l = sum(s[1] for s in states)
    return acc / l[:, None]


def _merge_exact(states):
    big_m = np.max([s[0] for s in states], axis=0)
    acc = sum(np.exp(s[0] - big_m)[:, None] * s[2] for s in states)
    l = sum(np.exp(s[0] - big_m) * s[1] for s in states)
    return acc / l[:, None]


def test_page_merge_fails_fp32_gate_exact_merge_passes():
    wl = inputs.CONFIGS[1]
    x = inputs.make_inputs(wl, "cpu", seed=0)
    ref, _ = oracle.ring_attention(inputs.to_f64(x.q), [inputs.to_f64(x.k_block(j)) for j in range(wl.num_blocks)],
                                   [inputs.to_f64(x.v_block(j)) for j in range(wl.num_blocks)], wl.q_pos0,
                                   [wl.kv_pos0(j) for j in range(wl.num_blocks)], wl.causal)
    ref = ref[0, :, 0, :]
    states = _block_states(x, wl)
    err_page = np.abs(_merge_without_common_max(states) - ref).max()
    err_exact = np.abs(_merge_exact(states) - ref).max()
    assert err_page > 1e-3, err_page
    assert err_exact < 1e-12, err_exact
