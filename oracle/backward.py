"""fp64 reference gradients of one device's share of ring attention (TEST
INFRASTRUCTURE ONLY; see the package docstring).

The pages train through the ring ("Ring Attention: Train 1M Tokens on 8GB GPUs
in 2026", section "Training Speed: The Numbers" (forward plus backward per
step), section "Gotchas and Failure Modes" (gradients flow backwards through
the ring) and section "What I Still Don't Understand" (the backward ring
direction)) but do not write the backward pass out.  Reading used: the exact gradient of the exact
forward, i.e. of O = softmax(scale Q K^T + mask) V, with respect to Q, K and V
for an upstream gradient dO.  In the ring each device produces dQ for its own
chunk and a contribution to dK_j, dV_j of every block j it received; those
contributions travel with the blocks and add up across devices.

Written from the definition, one query row at a time over the union of the
blocks (block order cannot matter): with P the softmax row,
  dV_c = sum_r P[r, c] dO_r
  dP[r, c] = <dO_r, v_c>
  dS[r, c] = P[r, c] (dP[r, c] - sum_c' P[r, c'] dP[r, c'])
  dQ_r = scale sum_c dS[r, c] k_c,   dK_c = scale sum_r dS[r, c] q_r
(the derivative of softmax: dS = P * (dP - rowsum(P * dP))).  Masked keys
have P = 0 and get no gradient from that row.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import _gather_blocks, default_scale, visible


def ring_attention_bwd(q, k_blocks: Sequence, v_blocks: Sequence, q_pos0: int, kv_pos0s: Sequence[int],
                       causal: bool, do, scale: float | None = None, pos_stride: int = 1):
    """Gradients of the ring-attention output of one device's chunk.

    q, do: [B, Sq, H, D]; k_blocks[j], v_blocks[j]: [B, Ck_j, H, D] (positions
    as in ring_attention).  Returns (dQ [B, Sq, H, D], dK list, dV list) in
    float64, dK[j] / dV[j] shaped like block j: this chunk's contribution.
    """
    q = np.asarray(q, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    bsz, sq, nh, d = q.shape
    if scale is None:
        scale = default_scale(d)
    nblk = len(k_blocks)
    kbs = [np.asarray(k, dtype=np.float64) for k in k_blocks]
    vbs = [np.asarray(v, dtype=np.float64) for v in v_blocks]
    dq = np.zeros_like(q)
    dk = [np.zeros_like(k) for k in kbs]
    dv = [np.zeros_like(v) for v in vbs]
    if nblk == 0 or sq == 0:
        return dq, dk, dv
    # keys of all blocks in one array, with their block index and row
    _, _, ps = _gather_blocks(kbs, vbs, kv_pos0s, pos_stride)
    order = sorted(range(nblk), key=lambda j: int(kv_pos0s[j]))  # the gather order
    kv_pos = np.concatenate(ps)
    vis = visible(int(q_pos0) + int(pos_stride) * np.arange(sq), kv_pos, causal)
    has = vis.any(axis=1)
    sizes = [kbs[j].shape[1] for j in order]
    starts = np.concatenate([[0], np.cumsum(sizes)])
    for b in range(bsz):
        for h in range(nh):
            kh = np.concatenate([kbs[j][b, :, h, :] for j in order], axis=0)
            vh = np.concatenate([vbs[j][b, :, h, :] for j in order], axis=0)
            qh = q[b, :, h, :]
            doh = do[b, :, h, :]
            s = np.where(vis, scale * (qh @ kh.T), -np.inf)
            p = np.zeros_like(s)
            m = s[has].max(axis=1, keepdims=True)
            e = np.exp(s[has] - m)
            p[has] = e / e.sum(axis=1, keepdims=True)
            dp = doh @ vh.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, :, h, :] = scale * (ds @ kh)
            dkh = scale * (ds.T @ qh)
            dvh = p.T @ doh
            for pos, j in enumerate(order):
                dk[j][b, :, h, :] = dkh[starts[pos]:starts[pos + 1]]
                dv[j][b, :, h, :] = dvh[starts[pos]:starts[pos + 1]]
    return dq, dk, dv


def delta(o, do):
    """Per-row D = sum_d dO * O ([B, H, Sq] from [B, Sq, H, D] tensors): the
    rowsum(P * dP) of the softmax derivative, since sum_c P dP = <dO, O>."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.transpose((o * do).sum(axis=3), (0, 2, 1))
