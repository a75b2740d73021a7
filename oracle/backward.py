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


def key_rows_bwd(q, do, k_blocks: Sequence, v_blocks: Sequence, q_pos0: int, kv_pos0s: Sequence[int], causal: bool,
                 key_rows: Sequence, scale: float | None = None, pos_stride: int = 1, chunk: int = 256):
    """dK and dV of chosen keys only, summed over every query row of q.

    The same gradient as ``ring_attention_bwd`` (module docstring), kept to
    the keys that are asked for, so that a long sequence can be checked
    without forming every key's gradient:
      dV_c = sum_r P[r, c] dO_r,   dK_c = scale sum_r P[r, c] (dP[r, c] - delta_r) q_r
    where P[r, :] is the softmax row of query r over ALL visible keys of all
    blocks, dP[r, c] = <dO_r, v_c> and delta_r = sum_c' P[r, c'] dP[r, c']
    over all of them too.  Query rows are taken `chunk` at a time (each
    chunk's full score rows, then its terms for the chosen keys), which
    bounds the memory; dK_c and dV_c are sums over rows, so the chunking
    changes nothing but the order of the additions.

    q, do: [B, Sq, H, D]; blocks and positions as in ``ring_attention_bwd``.
    key_rows: pairs (j, i), key i of block j (block indices as passed).
    Returns (dK [B, n, H, D], dV [B, n, H, D]) in float64, n = len(key_rows),
    in the order of key_rows.
    """
    q = np.asarray(q, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    bsz, sq, nh, d = q.shape
    if scale is None:
        scale = default_scale(d)
    kbs = [np.asarray(k, dtype=np.float64) for k in k_blocks]
    vbs = [np.asarray(v, dtype=np.float64) for v in v_blocks]
    n = len(key_rows)
    dv_dim = vbs[0].shape[3] if vbs else d
    dk = np.zeros((bsz, n, nh, d))
    dv = np.zeros((bsz, n, nh, dv_dim))
    if n == 0 or sq == 0:
        return dk, dv
    # every key of every block, in the order the blocks are given
    starts = np.concatenate([[0], np.cumsum([k.shape[1] for k in kbs])]).astype(np.int64)
    kv_pos = np.concatenate([int(kv_pos0s[j]) + int(pos_stride) * np.arange(kbs[j].shape[1], dtype=np.int64)
                             for j in range(len(kbs))])
    sel = np.array([starts[j] + i for j, i in key_rows], dtype=np.int64)
    q_pos = int(q_pos0) + int(pos_stride) * np.arange(sq, dtype=np.int64)
    for b in range(bsz):
        for h in range(nh):
            kh = np.concatenate([k[b, :, h, :] for k in kbs], axis=0)
            vh = np.concatenate([v[b, :, h, :] for v in vbs], axis=0)
            for r0 in range(0, sq, chunk):
                r1 = min(sq, r0 + chunk)
                vis = visible(q_pos[r0:r1], kv_pos, causal)
                has = vis.any(axis=1)
                if not has.any():
                    continue
                qc = q[b, r0:r1, h, :][has]
                doc = do[b, r0:r1, h, :][has]
                s = np.where(vis[has], scale * (qc @ kh.T), -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / e.sum(axis=1, keepdims=True)
                dp = doc @ vh.T
                delta_r = (p * dp).sum(axis=1, keepdims=True)
                p_sel = p[:, sel]
                ds_sel = p_sel * (dp[:, sel] - delta_r)
                dk[b, :, h, :] += scale * (ds_sel.T @ qc)
                dv[b, :, h, :] += p_sel.T @ doc
    return dk, dv
