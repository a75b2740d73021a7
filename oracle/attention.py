"""fp64 reference for one device's share of ring attention (TEST INFRASTRUCTURE ONLY).

Shapes follow the page's [sequence, heads, head_dim] layout with a leading
batch axis: q is [B, Sq, H, D]; each KV block is [B, Ck_j, H, D].  Every
input is converted to float64 (bf16 and fp32 values are exact in fp64).

The oracle deliberately ignores ring order: it gathers the keys of all blocks
in global-position order and evaluates each query row directly.  Exactness of
the ring (Abstract of "Ring Attention with Blockwise Transformers for
Near-Infinite Context") means the order in which blocks arrive cannot change
the answer, so an order-free definition is the right reference.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

LN2 = math.log(2.0)


def default_scale(head_dim: int) -> float:
    """1/sqrt(d_k): the softmax temperature of the attention equation in
    "Ring Attention: Train 1M Tokens on 8GB GPUs in 2026", section "Why
    Standard Attention Explodes Past 100K Tokens"; the same page's PyTorch
    section sets it to head_dim to the power -1/2."""
    return 1.0 / math.sqrt(head_dim)


def visible(q_pos: np.ndarray, kv_pos: np.ndarray, causal: bool) -> np.ndarray:
    """Boolean [n, N] visibility of key positions to query positions.

    The pages never define the causal mask.  Reading used (a language-model
    mask in global token positions, the plainest one consistent with the
    arXiv record's Abstract naming language modeling): key j is visible to
    query i iff kv_pos[j] <= q_pos[i], the diagonal included.  Positions are
    global, so a query chunk placed after a key block sees all of it.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    if not causal:
        return np.ones((q_pos.shape[0], kv_pos.shape[0]), dtype=bool)
    return kv_pos[None, :] <= q_pos[:, None]


def attention_rows(q, k, v, q_pos, kv_pos, causal: bool, scale: float):
    """Exact attention for a set of query rows against a set of keys.

    q: [n, D]; k, v: [N, D]; q_pos: [n]; kv_pos: [N].
    Returns (O [n, D], LSE [n]) in float64.

    Steps, per query row (materialising the full score row, as the attention
    definition does): s_j = scale * <q, k_j> for every key; keys that are not
    visible are dropped; M = max_j s_j; e_j = exp(s_j - M); L = sum_j e_j;
    O = (sum_j e_j v_j) / L; LSE = M + ln L (natural log).  A row with no
    visible key has O = 0 and LSE = -inf (convention; the pages never meet it).
    The max subtraction only keeps exp() in range; it cancels in O and is
    added back in LSE.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), -np.inf, dtype=np.float64)
    if n == 0 or k.shape[0] == 0:
        return out, lse
    s = scale * (q @ k.T)  # [n, N] full score rows
    vis = visible(q_pos, kv_pos, causal)
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    if not has.any():
        return out, lse
    s = s[has]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1, keepdims=True)
    out[has] = (e @ v) / l
    lse[has] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def _gather_blocks(k_blocks, v_blocks, kv_pos0s, pos_stride=1):
    """Concatenate KV blocks with their global key positions (block j's key i
    sits at kv_pos0s[j] + i * pos_stride)."""
    order = sorted(range(len(k_blocks)), key=lambda j: int(kv_pos0s[j]))
    ks, vs, ps = [], [], []
    for j in order:
        kb = np.asarray(k_blocks[j], dtype=np.float64)
        vb = np.asarray(v_blocks[j], dtype=np.float64)
        ks.append(kb)
        vs.append(vb)
        ps.append(int(kv_pos0s[j]) + int(pos_stride) * np.arange(kb.shape[1], dtype=np.int64))
    return ks, vs, ps


def ring_attention(q, k_blocks: Sequence, v_blocks: Sequence, q_pos0: int,
                   kv_pos0s: Sequence[int], causal: bool, scale: float | None = None,
                   rows: Sequence[int] | None = None, heads: Sequence[int] | None = None,
                   pos_stride: int = 1):
    """Exact attention of one device's query chunk over all KV blocks it receives.

    q: [B, Sq, H, D]; k_blocks[j], v_blocks[j]: [B, Ck_j, H, D]; block j holds
    global key positions kv_pos0s[j] + i * pos_stride for i = 0..Ck_j-1; query
    row r sits at global position q_pos0 + r * pos_stride.  pos_stride 1 is a
    contiguous chunk; pos_stride P the striped order (device i of P holds
    tokens i, i+P, ...), a reading of the Striped Attention entry of section
    "How Does This Compare to Other Long-Context Methods?" of "Ring Attention:
    Train 1M Tokens on 8GB GPUs in 2026".  The ring schedule of that page's
    section "Ring Attention: Partition Sequence Length, Not Batch" delivers
    every block exactly once, so the union of the blocks is the key set.
    Blocks may have different lengths (chunks of unequal length, the same
    page's FAQ).

    rows / heads restrict the evaluation to sampled query rows / heads.
    Returns (O [B, R, Hs, D], LSE [B, Hs, R]) in float64.
    """
    q = np.asarray(q)
    bsz, sq, nh, d = q.shape
    if scale is None:
        scale = default_scale(d)
    rows = np.arange(sq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(nh)) if heads is None else list(heads)
    ks, vs, ps = _gather_blocks(k_blocks, v_blocks, kv_pos0s, pos_stride)
    kv_pos = np.concatenate(ps) if ps else np.zeros((0,), np.int64)
    dv = vs[0].shape[3] if vs else d
    out = np.zeros((bsz, rows.shape[0], len(heads), dv))
    lse = np.full((bsz, len(heads), rows.shape[0]), -np.inf)
    q_pos = int(q_pos0) + int(pos_stride) * rows
    for b in range(bsz):
        for hi, h in enumerate(heads):
            qh = np.asarray(q[b, rows, h, :], dtype=np.float64)
            if ks:
                kh = np.concatenate([kb[b, :, h, :] for kb in ks], axis=0)
                vh = np.concatenate([vb[b, :, h, :] for vb in vs], axis=0)
            else:
                kh = np.zeros((0, d))
                vh = np.zeros((0, dv))
            o, ls = attention_rows(qh, kh, vh, q_pos, kv_pos, causal, scale)
            out[b, :, hi, :] = o
            lse[b, hi, :] = ls
    return out, lse


def partial_state(q, k_blocks: Sequence, v_blocks: Sequence, q_pos0: int,
                  kv_pos0s: Sequence[int], causal: bool, scale: float | None = None, pos_stride: int = 1):
    """The (m, l, acc) triple after a device has processed the given blocks.

    Closed form of the state named in the "Gotchas and Failure Modes" section
    of "Ring Attention: Train 1M Tokens on 8GB GPUs in 2026" (running max,
    running sum, weighted output), over the visible keys of the processed
    blocks S (positions as in ring_attention):
      m   = max_{j in S} s_j                     (natural-log score units)
      l   = sum_{j in S} exp(s_j - m)
      acc = sum_{j in S} exp(s_j - m) v_j        (unnormalised output)
    No visible key: m = -inf, l = 0, acc = 0.  Consequently acc / l is the
    attention output over S and m + ln l its log-sum-exp.
    Returns m [B, H, Sq], l [B, H, Sq], acc [B, H, Sq, D] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, sq, nh, d = q.shape
    if scale is None:
        scale = default_scale(d)
    ks, vs, ps = _gather_blocks(k_blocks, v_blocks, kv_pos0s, pos_stride)
    dv = vs[0].shape[3] if vs else d
    m = np.full((bsz, nh, sq), -np.inf)
    l = np.zeros((bsz, nh, sq))
    acc = np.zeros((bsz, nh, sq, dv))
    if not ks:
        return m, l, acc
    kv_pos = np.concatenate(ps)
    vis = visible(int(q_pos0) + int(pos_stride) * np.arange(sq), kv_pos, causal)
    has = vis.any(axis=1)
    for b in range(bsz):
        for h in range(nh):
            kh = np.concatenate([kb[b, :, h, :] for kb in ks], axis=0)
            vh = np.concatenate([vb[b, :, h, :] for vb in vs], axis=0)
            s = np.where(vis, scale * (q[b, :, h, :] @ kh.T), -np.inf)
            mh = s[has].max(axis=1)
            e = np.exp(s[has] - mh[:, None])
            m[b, h, has] = mh
            l[b, h, has] = e.sum(axis=1)
            acc[b, h, has, :] = e @ vh
    return m, l, acc
