"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle on
the same inputs, compare at the stated tolerances."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra

# Tolerances.  fp32 inputs: max |dO| <= 1e-5 and max |dLSE| <= 1e-5.  bf16
# inputs: max |dO| <= 2e-2 and |dLSE| <= 1e-3 * max(1, |LSE|) (relative, with
# a floor at 1 so rows whose LSE is near 0 are held to 1e-3 absolute); and,
# because |O| is small when the softmax is flat, max |dO| <= 1e-2 * max |O|.
TOL = {
    "f32": dict(o_abs=1e-5, lse_abs=1e-5),
    "bf16": dict(o_abs=2e-2, lse_rel=1e-3, o_scaled=1e-2),
}


def cuda():
    return torch.device("cuda:0")


def ring_positions(wl: inputs.Workload, order):
    return [wl.kv_pos0(j) for j in order]


def run_hip(x: inputs.Inputs, order=None, perblock=False, out_dtype=None):
    wl = x.wl
    order = list(range(wl.num_blocks)) if order is None else list(order)
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    o, lse = ra.ring_forward(x.q, kb, vb, ring_positions(wl, order), q_pos0=wl.q_pos0, causal=wl.causal,
                             perblock=perblock, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


def oracle_ref(x: inputs.Inputs, rows=None, heads=None):
    """Oracle O [B, R, Hs, D] and LSE [B, Hs, R] on the exact input values,
    one head at a time (keeps the fp64 copies small)."""
    wl = x.wl
    heads = list(range(wl.heads)) if heads is None else list(heads)
    rows = np.arange(wl.q_len) if rows is None else np.asarray(rows)
    outs, lses = [], []
    for h in heads:
        q = inputs.to_f64(x.q[:, :, h:h + 1, :])
        kb = [inputs.to_f64(x.k_block(j)[:, :, h:h + 1, :]) for j in range(wl.num_blocks)]
        vb = [inputs.to_f64(x.v_block(j)[:, :, h:h + 1, :]) for j in range(wl.num_blocks)]
        o, lse = oracle.ring_attention(q, kb, vb, wl.q_pos0, [wl.kv_pos0(j) for j in range(wl.num_blocks)],
                                       wl.causal, rows=rows)
        outs.append(o)
        lses.append(lse)
    return np.concatenate(outs, axis=2), np.concatenate(lses, axis=1)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what=""):
    """Element-wise comparison at the tolerance of the input dtype.  o_gpu /
    lse_gpu are numpy float64 arrays already restricted to the rows/heads of
    the reference.  Returns the error summary."""
    tol = TOL[dtype]
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: LSE finiteness differs"
    err_o = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    d_lse = np.abs(lse_gpu[fin] - lse_ref[fin])
    out = {"max_abs_o": err_o}
    if dtype == "f32":
        err_l = float(d_lse.max()) if d_lse.size else 0.0
        out["max_abs_lse"] = err_l
        assert err_o <= tol["o_abs"], f"{what}: max|dO| {err_o:.3e} > {tol['o_abs']}"
        assert err_l <= tol["lse_abs"], f"{what}: max|dLSE| {err_l:.3e} > {tol['lse_abs']}"
    else:
        rel = d_lse / np.maximum(1.0, np.abs(lse_ref[fin])) if d_lse.size else np.zeros(1)
        scale = float(np.max(np.abs(o_ref))) if o_ref.size else 0.0
        out.update(max_rel_lse=float(rel.max()), scaled_o=err_o / scale if scale > 0 else 0.0)
        assert err_o <= tol["o_abs"], f"{what}: max|dO| {err_o:.3e} > {tol['o_abs']}"
        assert rel.max() <= tol["lse_rel"], f"{what}: LSE rel err {rel.max():.3e} > {tol['lse_rel']}"
        if scale > 0:
            assert err_o <= tol["o_scaled"] * scale, f"{what}: max|dO|/max|O| {err_o / scale:.3e}"
    return out


def gpu_rows(o, lse, rows=None, heads=None):
    """Select rows/heads of GPU outputs as float64 numpy (O [B,R,Hs,D], LSE [B,Hs,R])."""
    o = o.float()
    if rows is not None:
        idx = torch.as_tensor(rows, device=o.device, dtype=torch.long)
        o = o.index_select(1, idx)
        lse = lse.index_select(2, idx)
    if heads is not None:
        hidx = torch.as_tensor(heads, device=o.device, dtype=torch.long)
        o = o.index_select(2, hidx)
        lse = lse.index_select(1, hidx)
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def small(dtype="bf16", heads=2, d=128, q_len=300, kv_len=200, p=4, causal=True, q_idx=2, in_scale=1.0):
    return inputs.Workload(f"test {dtype} H{heads} D{d} Q{q_len} P{p}x{kv_len} c{int(causal)} q{q_idx}", dtype,
                           heads, d, q_len, kv_len, p, causal, q_idx, in_scale=in_scale)


def lse_natural_from_state(m, l):
    with np.errstate(divide="ignore"):
        return np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)


__all__ = ["TOL", "cuda", "run_hip", "oracle_ref", "compare", "gpu_rows", "small", "math"]
