#!/usr/bin/env python3
"""Benchmark: one device's share of a causal ring-attention forward on one MI355X.

A step is one whole ring pass (every KV block of the ring attended and merged,
O and LSE written) over the workload's synthetic inputs, which are resident in
HBM before timing starts.  Default workload: 16 heads, head_dim 128, local
query chunk 131072 rows (512K tokens over a ring of 4), 4 KV blocks of 131072
keys, causal with the chunk at ring index 3, bf16 in / fp32 accumulate.

Unless --no-backward, the same line carries a `backward` object: the
gradient pass through the ring (delta, dQ of the chunk and the chunk's dK/dV
contribution for every block) timed on the same inputs with the forward's O
and LSE, in algorithmic TFLOP/s (10*B*H*D*(visible pairs): the five products
S, dP, dQ, dK, dV), with dQ checked against the oracle on sampled rows and the
sums of dK and dV over all keys checked against their closed forms.

Unless --no-ffn, it also carries `ffn`: the blockwise feedforward of the
1.3B model's layer (d 2048, d_ff 8192, tanh GELU) over the same 128K-row
chunk in 16K-row blocks, in TFLOP/s of its two products (4*rows*d*d_ff),
with sampled rows checked against the oracle, and beside it torch's own path
for the same blockwise network (hipBLASLt GEMMs with bias, then GELU) as a
stated baseline.

Unless --no-workloads (default workload only), `workloads` carries timings of
the other three workloads: the 32K chunk against 8 blocks, the 1M-token pass
over 128 devices (8K chunk, 128 blocks: two fused launches), and the 32K
chunk with its blocks streamed from pinned host memory (T_streamed,
T_resident, T_copy, overlap efficiency, fraction of the H2D rate).

Prints ONE JSON line.  `value` is causal-adjusted TFLOP/s: 4*B*H*D*(visible
query-key pairs) per step over the measured step time.  `roofline` prices the
fused attention kernel's live-measured duration (HIP events on the launch
stream) against the bf16 dense MFMA peak.  `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]
       [--perblock] [--no-cpu-baseline] [--traffic-calib] [--no-backward] [--bwd-steps K] [--no-ffn]
       [--no-workloads]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal-adjusted attention TFLOP/s on 1 MI355X; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 flop/clk/CU x 2.4 GHz (AMD's published 2.5 PF)
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = [os.path.join(ROOT, "long_context_exact_blockwise_amd", "csrc", f)
              for f in ("attn_bf16.hip", "attn_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_fused_causal_q131072_p4_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_bf16_fused_causal_q131072_p4_stall_counters.txt")


def visible_pairs(wl) -> int:
    """Query-key pairs with the key visible to the query, one head: a key at
    position p is visible to a query at position t iff p <= t (causal), all
    pairs otherwise."""
    total = 0
    q0, q1 = wl.q_pos0, wl.q_pos0 + wl.q_len - 1
    for j in range(wl.num_blocks):
        k0 = wl.kv_pos0(j)
        k1 = k0 + wl.kv_len - 1
        if not wl.causal:
            total += wl.q_len * wl.kv_len
            continue
        # rows t >= k1 see the whole block
        full_from = max(q0, k1)
        if full_from <= q1:
            total += (q1 - full_from + 1) * wl.kv_len
        # rows k0 <= t < k1 see t - k0 + 1 keys
        lo, hi = max(q0, k0), min(q1, k1 - 1)
        if hi >= lo:
            n = hi - lo + 1
            total += n * (lo - k0 + 1) + n * (n - 1) // 2
    return total


def flops(wl) -> int:
    return 4 * wl.batch * wl.heads * wl.head_dim * visible_pairs(wl)


def kernel_hash() -> str:
    """Hash of the fused kernel's sources and its per-source build flags."""
    from long_context_exact_blockwise_amd.build import SOURCE_FLAGS
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(repr(SOURCE_FLAGS.get("attn_bf16.hip", [])).encode())
    return h.hexdigest()[:16]


def source_hash(files, flags) -> str:
    """Hash of kernel sources (names under the package's csrc/) and their
    build flags, the tag each profile summary carries for the build it was
    taken on."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "long_context_exact_blockwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(repr(flags).encode())
    return h.hexdigest()[:16]


def backward_hash() -> str:
    from long_context_exact_blockwise_amd.build import SPLIT
    return source_hash(("attn_bwd.hip", "attn_common.h"), SPLIT["attn_bwd.hip"])


def feedforward_hash() -> str:
    from long_context_exact_blockwise_amd.build import SOURCE_FLAGS
    return source_hash(("ffn_bf16.hip", "attn_common.h"), SOURCE_FLAGS.get("ffn_bf16.hip", []))


def read_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    missing or taken on a different kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256_16") != kernel_hash():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def read_mfma_busy():
    """Fraction of SIMD cycles the matrix cores were busy under the fused
    kernel, from the committed rocprofv3 counter summary:
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).  None
    when the file is missing or was taken on a different kernel source."""
    try:
        kv = {}
        src = None
        with open(COUNTERS_FILE) as f:
            for line in f:
                if line.startswith("kernel_source_sha256_16:"):
                    src = line.split(":", 1)[1].strip()
                parts = line.split()
                if len(parts) == 2 and parts[0].isupper():
                    kv[parts[0]] = float(parts[1])
        if src != kernel_hash():
            return None
        return kv["SQ_VALU_MFMA_BUSY_CYCLES"] / (kv["GRBM_GUI_ACTIVE"] / 8 * 1024)
    except (OSError, KeyError, ValueError, ZeroDivisionError):
        return None


def probe_peak(dev, iters: int = 200000, reps: int = 2, random_operands: bool = False, lds_reads: int = 0) -> float:
    """bf16 MFMA rate the part sustains under load (TFLOP/s): the library's
    MFMA-only probe on every CU (four 512-thread groups per CU, four waves per
    SIMD, ~50 ms per launch), best of `reps`.  Its operands are a fixed
    pattern of small values, or with `random_operands` seeded N(0, 1) bf16
    values (more bits toggle per product: more power, a lower clock).  With
    `lds_reads` (4, 8 or 16; random operands) every product's first operand
    comes from LDS, lds_reads / 16 KiB per product and wave, and `iters`
    counts products / 4 as for the other forms."""
    import torch
    from long_context_exact_blockwise_amd import ringattn as ra
    wgs = 4 * 256
    out = torch.empty(wgs * ra.PROBE_THREADS, dtype=torch.float32, device=dev)
    ops = None
    if random_operands or lds_reads:
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        ops = torch.randn(wgs * ra.PROBE_THREADS * ra.PROBE_OPERANDS_PER_THREAD, generator=g, device=dev,
                          dtype=torch.float32).to(torch.bfloat16)

    def launch(n):
        if lds_reads:
            ra.ringattn_probe_mfma_lds(ops, out, wgs, max(1, n // 4), lds_reads)
        elif ops is None:
            ra.ringattn_probe_mfma(out, wgs, n)
        else:
            ra.ringattn_probe_mfma_data(ops, out, wgs, n)
    launch(1000)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch(iters)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if lds_reads:
            f = wgs * (ra.PROBE_THREADS // 64) * max(1, iters // 4) * ra.PROBE_LDS_FLOP_PER_ITER_PER_WAVE
        else:
            f = wgs * (ra.PROBE_THREADS // 64) * iters * ra.PROBE_FLOP_PER_ITER_PER_WAVE
        best = max(best, f / (ms * 1e-3) / 1e12)
    return best


def bwd_flops(wl) -> int:
    return 10 * wl.batch * wl.heads * wl.head_dim * visible_pairs(wl)


def backward_measure(x, wl, kb, vb, pos, o, lse, steps, warmup, sample_heads):
    """Time the ring backward and check it at full size: dQ on sampled rows
    against the oracle; sum_c dK_c = 0 and sum_c dV_c = sum_r dO_r (every row
    sees a key) per head, in fp64 on the host."""
    import numpy as np
    import torch
    import oracle
    from long_context_exact_blockwise_amd import inputs
    from long_context_exact_blockwise_amd import ringattn as ra
    dev = x.q.device
    do = inputs.make_grad(wl, dev, seed=1)
    desc = ra.make_desc(x.q, kb[0], o, q_pos0=wl.q_pos0, causal=wl.causal)
    delta = torch.empty((wl.batch, wl.heads, wl.q_len), dtype=torch.float32, device=dev)
    dq = torch.empty((wl.batch, wl.q_len, wl.heads, wl.head_dim), dtype=torch.float32, device=dev)
    dk = [torch.zeros((wl.batch, wl.kv_len, wl.heads, wl.head_dim), dtype=torch.float32, device=dev) for _ in kb]
    dv = [torch.zeros_like(t) for t in dk]

    def step():
        ra.ringattn_ring_bwd(desc, x.q, kb, vb, pos, o, do, lse, delta, dq, dk, dv)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # one clean pass for the checks
    for t in dk + dv:
        t.zero_()
    step()
    torch.cuda.synchronize()
    f = bwd_flops(wl)
    # three windows of consecutive rows (first, seeded, last): the oracle's
    # cost is in the keys, so a window costs what one row does
    r0 = int(np.random.default_rng(2).integers(4, wl.q_len - 12))
    windows = [(0, 4), (r0, r0 + 8), (wl.q_len - 4, wl.q_len)]
    rows = [r for a, b in windows for r in range(a, b)]
    rows_np = np.asarray(rows)
    q_host, k_host, v_host, do_host = x.q.cpu(), x.k.cpu(), x.v.cpu(), do.cpu()
    dq_host = dq.cpu().double().numpy()
    fro_num = fro_den = 0.0
    inv_err = 0.0
    porder = list(range(wl.num_blocks))
    for h in sample_heads:
        qh = q_host[:, rows_np, h:h + 1, :].float().double().numpy()
        doh = do_host[:, rows_np, h:h + 1, :].float().double().numpy()
        kbh = [k_host[:, j * wl.kv_len:(j + 1) * wl.kv_len, h:h + 1, :].float().double().numpy() for j in porder]
        vbh = [v_host[:, j * wl.kv_len:(j + 1) * wl.kv_len, h:h + 1, :].float().double().numpy() for j in porder]
        i = 0
        for a, b in windows:  # dQ rows are independent: each window at its own positions
            rq, _, _ = oracle.ring_attention_bwd(qh[:, i:i + b - a], kbh, vbh, wl.q_pos0 + a,
                                                 [wl.kv_pos0(j) for j in porder], wl.causal, doh[:, i:i + b - a])
            g = dq_host[:, a:b, h:h + 1, :]
            fro_num += float(((g - rq) ** 2).sum())
            fro_den += float((rq ** 2).sum())
            i += b - a
        sdk = sum(t[:, :, h].double().sum(dim=1) for t in dk).cpu().numpy()
        sdv = sum(t[:, :, h].double().sum(dim=1) for t in dv).cpu().numpy()
        sdo = do_host[:, :, h].double().sum(dim=1).numpy()
        mag = sum(t[:, :, h].double().abs().sum(dim=1) for t in dv).cpu().numpy()
        inv_err = max(inv_err, float(np.abs(sdv - sdo).max() / mag.max()),
                      float(np.abs(sdk).max() / sum(t[:, :, h].double().abs().sum(dim=1) for t in dk).max().item()))
    fro = (fro_num / fro_den) ** 0.5 if fro_den else 0.0
    ok = fro <= 5e-3 and inv_err <= 1e-3
    return {
        "ms_per_step": ms, "steps": steps, "warmup": warmup, "value": f / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "pct_of_bf16_peak": 100.0 * f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "algorithmic_flop_per_step": f,
        "kernels": "bwd_dq_kernel + bwd_dkdv_kernel per block, bwd_delta_kernel, fill_zero_kernel",
        "parity_sampled": {"dq_rows": len(rows) * len(sample_heads), "dq_rel_fro": fro,
                           "sum_dk_dv_invariants_rel": inv_err, "pass": bool(ok)},
    }


def ffn_measure(dev, steps, warmup):
    """Time the blockwise feedforward at its workload and check sampled rows
    against the oracle (rows are independent)."""
    import numpy as np
    import torch
    import oracle
    from long_context_exact_blockwise_amd import inputs
    from long_context_exact_blockwise_amd import ringattn as ra
    wl = inputs.FFN_CONFIG
    x, w1, b1, w2, b2 = inputs.make_ffn_inputs(wl.rows, wl.d_model, wl.d_ff, dev, seed=0)
    y = torch.empty_like(x)
    ws = torch.empty((wl.block_rows, wl.d_ff), dtype=torch.bfloat16, device=dev)
    desc = ra.ffn_desc(x, w1, y, wl.block_rows)
    # torch's own path for the same blockwise network, a stated baseline:
    # hipBLASLt GEMMs with the bias, then a separate tanh GELU
    import torch.nn.functional as F
    y_t = torch.empty_like(x)
    br = wl.block_rows

    def ours():
        ra.ringattn_ffn_fwd(desc, x, w1, b1, w2, b2, y, ws)

    def torch_pass():
        for r0 in range(0, wl.rows, br):
            hid = F.gelu(F.linear(x[r0:r0 + br], w1, b1), approximate="tanh")
            y_t[r0:r0 + br] = F.linear(hid, w2, b2)

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps
    for _ in range(warmup):
        ours()
        torch_pass()
    torch.cuda.synchronize()
    # alternate the two paths so that both see the same clock and heat
    rounds = [(timed(ours), timed(torch_pass)) for _ in range(3)]
    ms = float(np.median([a for a, _ in rounds]))
    ms_t = float(np.median([b for _, b in rounds]))
    f = 4 * wl.rows * wl.d_model * wl.d_ff
    rows = inputs.sample_rows(wl.rows, extra=14, seed=3)
    idx = torch.as_tensor(rows, device=dev)
    f64 = lambda t: t.float().double().cpu().numpy()  # noqa: E731
    ref = oracle.blockwise_ffn(f64(x.index_select(0, idx)), f64(w1), f64(b1), f64(w2), f64(b2))
    g = f64(y.index_select(0, idx))
    fro = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(g - ref)) / np.max(np.abs(ref)))
    return {
        "workload": wl.name, "ms_per_step": ms, "steps": steps, "value": f / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "pct_of_bf16_peak": 100.0 * f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "algorithmic_flop_per_step": f,
        "kernels": "gemm_bt_kernel<gelu> + gemm_bt_kernel<plain> per block",
        "parity_sampled": {"rows": len(rows), "rel_fro": fro, "max_abs_over_max": mx,
                           "pass": bool(fro <= 5e-3 and mx <= 2e-2)},
        "rounds_ms": [round(a, 4) for a, _ in rounds],
        "torch_hipblaslt_baseline": {"ms_per_step": ms_t, "value": f / (ms_t * 1e-3) / 1e12, "unit": "TFLOP/s",
                                     "rounds_ms": [round(b, 4) for _, b in rounds],
                                     "path": "per block: F.linear (hipBLASLt, bias) -> F.gelu(tanh) -> F.linear"},
        "timing": f"median of 3 rounds of {steps} passes, the two paths alternating",
    }


def _duration(sec: float) -> str:
    """Seconds as a short human duration with two significant digits."""
    for unit, div in (("h", 3600.0), ("min", 60.0), ("s", 1.0)):
        if sec >= div or unit == "s":
            return f"{sec / div:.2g} {unit}"


def _single_core_oracle(x, wl, heads, rows):
    """The same oracle on one core (BLAS limited to one thread): a smaller
    sample of the same rows, in the same unit."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    pos = [wl.kv_pos0(j) for j in range(wl.num_blocks)]
    k_host, v_host, q_host = x.k.cpu(), x.v.cpu(), x.q.cpu()
    t = 0.0
    n_vis = 0
    with threadpool_limits(limits=1):
        for h in heads:
            q64 = q_host[:, :, h:h + 1, :].float().double().numpy()
            kb = [k_host[:, j * wl.kv_len:(j + 1) * wl.kv_len, h:h + 1, :].float().double().numpy()
                  for j in range(wl.num_blocks)]
            vb = [v_host[:, j * wl.kv_len:(j + 1) * wl.kv_len, h:h + 1, :].float().double().numpy()
                  for j in range(wl.num_blocks)]
            t0 = time.perf_counter()
            oracle.ring_attention(q64, kb, vb, wl.q_pos0, pos, wl.causal, rows=np.asarray(rows))
            t += time.perf_counter() - t0
    for r in rows:
        tq = wl.q_pos0 + int(r)
        for j in range(wl.num_blocks):
            n_vis += wl.kv_len if not wl.causal else max(0, min(wl.kv_len, tq - wl.kv_pos0(j) + 1))
    f = 4 * wl.head_dim * n_vis * len(heads)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": t,
            "sample": f"{len(rows)} of the same rows x {len(heads)} head, BLAS on one thread"}


def cpu_baseline(x, wl, o, lse, heads=None, extra_rows=94):
    """Time the fp64 oracle on sampled rows of every head; also check those
    rows against the GPU output at the bf16 tolerances."""
    import numpy as np
    import oracle
    from long_context_exact_blockwise_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    heads = list(range(wl.heads)) if heads is None else heads
    rows = inputs.sample_rows(wl.q_len, extra=extra_rows, seed=1)
    rows_np = np.asarray(rows)
    k_host = x.k.cpu()
    v_host = x.v.cpu()
    q_host = x.q.cpu()
    o_host = o.float().cpu().numpy()
    lse_host = lse.cpu().numpy()
    t_oracle = 0.0
    err_o = 0.0
    err_l = 0.0
    scale_o = 0.0
    pos = [wl.kv_pos0(j) for j in range(wl.num_blocks)]
    for h in heads:
        q64 = q_host[:, :, h:h + 1, :].float().double().numpy()
        kb = [k_host[:, j * wl.kv_len:(j + 1) * wl.kv_len, h:h + 1, :].float().double().numpy()
              for j in range(wl.num_blocks)]
        vb = [v_host[:, j * wl.kv_len:(j + 1) * wl.kv_len, h:h + 1, :].float().double().numpy()
              for j in range(wl.num_blocks)]
        t0 = time.perf_counter()
        ro, rl = oracle.ring_attention(q64, kb, vb, wl.q_pos0, pos, wl.causal, rows=rows_np)
        t_oracle += time.perf_counter() - t0
        go = o_host[:, rows_np, h:h + 1, :]
        gl = lse_host[:, h:h + 1, rows_np]
        err_o = max(err_o, float(np.abs(go - ro).max()))
        err_l = max(err_l, float((np.abs(gl - rl) / np.maximum(1.0, np.abs(rl))).max()))
        scale_o = max(scale_o, float(np.abs(ro).max()))
    # algorithmic flops of the sampled rows (visible keys per row x 4D)
    n_vis = 0
    for r in rows:
        t = wl.q_pos0 + r
        for j in range(wl.num_blocks):
            k0 = wl.kv_pos0(j)
            n_vis += wl.kv_len if not wl.causal else max(0, min(wl.kv_len, t - k0 + 1))
    f = 4 * wl.head_dim * n_vis * len(heads)
    value = f / t_oracle / 1e12
    per_pair = t_oracle / (n_vis * len(heads))
    base = {
        "value": value, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{len(rows)} query rows (first, last, {extra_rows} seeded) x {len(heads)} heads of the same workload, "
                  f"fp64 NumPy, {t_oracle:.1f} s; full-workload extrapolation "
                  f"{_duration(per_pair * visible_pairs(wl) * wl.heads * wl.batch)}",
        "seconds": t_oracle,
        "single_core": _single_core_oracle(x, wl, heads[:1], rows_np[:max(2, len(rows_np) // 8)]),
    }
    tol_ok = err_o <= 2e-2 and err_l <= 1e-3 and (scale_o == 0 or err_o <= 1e-2 * scale_o)
    parity = {"rows": len(rows) * len(heads), "max_abs_o": err_o, "max_rel_lse": err_l,
              "max_abs_o_over_max_o": err_o / scale_o if scale_o else 0.0, "pass": bool(tol_ok)}
    return base, parity


def streamed_overlap(x, kb, vb, pos, o, lse, desc, ws, hk, hv, stage_k, stage_v, t_str, steps):
    """Overlap of the host-streamed pass: its time t_str (s) against the
    device-resident per-block pass and the H2D copies alone."""
    import torch
    from long_context_exact_blockwise_amd import ringattn as ra

    def resident():
        ra.ringattn_ring_fwd(desc, x.q, kb, vb, pos, o, lse, *ws)
    for _ in range(2):
        resident()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        resident()
    torch.cuda.synchronize()
    t_res = (time.perf_counter() - t1) / steps
    nbytes = sum(t.numel() * t.element_size() for t in hk + hv)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        for i in range(len(hk)):
            stage_k[i % 2].copy_(hk[i], non_blocking=True)
            stage_v[i % 2].copy_(hv[i], non_blocking=True)
    torch.cuda.synchronize()
    t_copy = (time.perf_counter() - t1) / steps
    eta = (t_res + t_copy - t_str) / min(t_res, t_copy)
    return {
        "t_streamed_ms": t_str * 1e3, "t_resident_ms": t_res * 1e3, "t_copy_ms": t_copy * 1e3,
        "h2d_GBps": nbytes / t_copy / 1e9, "h2d_bytes": nbytes,
        "fraction_of_h2d_bw": (nbytes / t_str) / (nbytes / t_copy),
        "overlap_efficiency": max(0.0, min(1.0, eta)),
        "note": "overlap = (T_resident + T_copy - T_streamed) / min(T_resident, T_copy); the PCIe-inclusive "
                "rate is `value`; fraction_of_h2d_bw = achieved H2D rate during the streamed pass over the "
                "copy-only rate",
    }


def workload_summary(dev, cfg: int, steps: int = 5, warmup: int = 2) -> dict:
    """Timings only for another workload: the fused ring pass (its own
    inputs, generated here), or for the host-streamed workload the
    streamed per-block pass with its overlap figures."""
    import torch
    from long_context_exact_blockwise_amd import inputs
    from long_context_exact_blockwise_amd import ringattn as ra
    wl = inputs.CONFIGS[cfg]
    x = inputs.make_inputs(wl, dev, seed=0)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o = torch.empty_like(x.q)
    lse = torch.empty((wl.batch, wl.heads, wl.q_len), dtype=torch.float32, device=dev)
    perblock = wl.host_streamed
    desc = ra.make_desc(x.q, kb[0], o, q_pos0=wl.q_pos0, causal=wl.causal,
                        flags=ra.RA_FLAG_PERBLOCK if perblock else 0)
    ws = ra.state_buffers(desc, dev) if (perblock or len(kb) > ra.RA_FUSED_MAX_BLOCKS) else (None, None, None)
    if wl.host_streamed:
        hk = [t.cpu().pin_memory() for t in kb]
        hv = [t.cpu().pin_memory() for t in vb]
        stage_k = [torch.empty_like(kb[0]).contiguous() for _ in range(2)]
        stage_v = [torch.empty_like(vb[0]).contiguous() for _ in range(2)]
        copy_stream = torch.cuda.Stream()
        hdesc = ra.make_desc(x.q, hk[0], o, q_pos0=wl.q_pos0, causal=wl.causal)

        def step():
            ra.ringattn_ring_fwd(hdesc, x.q, hk, hv, pos, o, lse, *ws, kv_on_host=True, stage_k=stage_k,
                                 stage_v=stage_v, copy_stream=copy_stream)
    else:
        def step():
            ra.ringattn_ring_fwd(desc, x.q, kb, vb, pos, o, lse, *ws)
    for _ in range(warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    ev_ms = sorted(a.elapsed_time(b) for a, b in evs)
    f = flops(wl)
    out = {
        "workload": wl.name, "path": "host-streamed per-block" if perblock else "fused", "steps": steps,
        "ms_per_step": ms, "kernel_ms_median": ev_ms[len(ev_ms) // 2], "kernel_ms_min": ev_ms[0],
        "value": f / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "pct_of_bf16_peak": 100.0 * f / (ms * 1e-3) / 1e12 /
        PEAK_BF16_TFLOPS, "algorithmic_flop_per_step": f,
        "launches_per_step": None if perblock else -(-len(kb) // ra.RA_FUSED_MAX_BLOCKS),
        "outputs_finite": bool(torch.isfinite(o.float()).all().item()),
    }
    if wl.host_streamed:
        out["host_streamed"] = streamed_overlap(x, kb, vb, pos, o, lse, desc, ws, hk, hv, stage_k, stage_v,
                                                ms * 1e-3, steps)
    del x, kb, vb, o, lse, ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--perblock", action="store_true", help="per-block path instead of the fused kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--bwd-steps", type=int, default=3)
    ap.add_argument("--no-ffn", action="store_true", help="skip the feedforward measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the timings of the other workloads (32K chunk, 1M tokens / 128, host-streamed)")
    ap.add_argument("--traffic-calib", action="store_true",
                    help="also run one 1 GiB plain copy kernel (byte-counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one device's share of the ring on ONE GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the inter-device ring is out of scope.", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_exact_blockwise_amd import inputs
    from long_context_exact_blockwise_amd import ringattn as ra

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ra.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    wl = inputs.CONFIGS[args.workload]
    x = inputs.make_inputs(wl, dev, seed=0)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    kb = [x.k_block(j) for j in order]
    vb = [x.v_block(j) for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o = torch.empty_like(x.q)
    lse = torch.empty((wl.batch, wl.heads, wl.q_len), dtype=torch.float32, device=dev)
    perblock = args.perblock or wl.host_streamed
    desc = ra.make_desc(x.q, kb[0], o, q_pos0=wl.q_pos0, causal=wl.causal,
                        flags=ra.RA_FLAG_PERBLOCK if perblock else 0)
    ws = ra.state_buffers(desc, dev) if (perblock or len(kb) > ra.RA_FUSED_MAX_BLOCKS) else (None, None, None)

    extra = {}
    if wl.host_streamed:
        hk = [t.cpu().pin_memory() for t in kb]
        hv = [t.cpu().pin_memory() for t in vb]
        stage_k = [torch.empty_like(kb[0]).contiguous() for _ in range(2)]
        stage_v = [torch.empty_like(vb[0]).contiguous() for _ in range(2)]
        copy_stream = torch.cuda.Stream()
        hdesc = ra.make_desc(x.q, hk[0], o, q_pos0=wl.q_pos0, causal=wl.causal)

        def step():
            ra.ringattn_ring_fwd(hdesc, x.q, hk, hv, pos, o, lse, *ws, kv_on_host=True, stage_k=stage_k,
                                 stage_v=stage_v, copy_stream=copy_stream)
    else:
        def step():
            ra.ringattn_ring_fwd(desc, x.q, kb, vb, pos, o, lse, *ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps, events around each for the kernel
    # durations (same stream as the launches: torch's current stream).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ev_ms = [a.elapsed_time(b) for a, b in evs]
    kern_ms = sum(ev_ms) / len(ev_ms)
    f = flops(wl)
    value = f / (ms_step * 1e-3) / 1e12
    achieved = f / (kern_ms * 1e-3) / 1e12
    finite = bool(torch.isfinite(o.float()).all().item())

    if wl.host_streamed:
        extra["host_streamed"] = streamed_overlap(x, kb, vb, pos, o, lse, desc, ws, hk, hv, stage_k, stage_v,
                                                  ms_step * 1e-3, args.steps)

    probed = probe_peak(dev) if wl.dtype == "bf16" else None
    probed_rand = probe_peak(dev, iters=100000, random_operands=True) if wl.dtype == "bf16" else None
    probed_lds = probe_peak(dev, iters=100000, lds_reads=16) if wl.dtype == "bf16" else None

    if args.traffic_calib:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        ra.ringattn_probe_copy(src, dst, n)
        torch.cuda.synchronize()
        del src, dst

    # the committed counter summary covers the fused kernel on the default workload only
    traffic = read_traffic() if (not perblock and args.workload == 3) else None
    kname = "attn_bf16_kernel" if wl.dtype == "bf16" else "attn_f32_kernel"
    roofline = {
        "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
        "hbm_GBps": (traffic / (kern_ms * 1e-3) / 1e9) if traffic else None,
        "hbm_GBps_note": "traffic (calibrated rocprofv3 FETCH_SIZE + WRITE_SIZE of the same kernel source) "
                         "over this run's kernel time",
        "mfma_busy": read_mfma_busy() if traffic else None,
        "mfma_busy_note": "rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) "
                          "from the committed counter summary of the same kernel source",
        "kernel": kname + (" (fused ring pass)" if not perblock else " (per block)"),
        "launches_per_step": 1 if (not perblock and len(kb) <= ra.RA_FUSED_MAX_BLOCKS) else None,
        "algorithmic_flop_per_step": f,
        "probed_peak": probed,
        "frac_of_probed": (achieved / probed) if probed else None,
        "probed_peak_note": "bf16 MFMA rate measured on this part under load by ringattn_probe_mfma "
                            "(MFMA-only kernel on every CU); peak is the published 2.5 PF figure",
        "probed_peak_random_operands": probed_rand,
        "frac_of_probed_random_operands": (achieved / probed_rand) if probed_rand else None,
        "probed_peak_random_operands_note": "the same probe with seeded N(0, 1) bf16 operands "
                                            "(ringattn_probe_mfma_data): the rate the part sustains on data like "
                                            "the attention's, where power limits the clock",
        "probed_peak_random_operands_lds_1k": probed_lds,
        "frac_of_probed_random_operands_lds_1k": (achieved / probed_lds) if probed_lds else None,
        "probed_peak_random_operands_lds_1k_note": "the random-operand probe with every product's first "
                                                   "operand read from LDS, 1 KiB per product and wave "
                                                   "(ringattn_probe_mfma_lds, lds_reads 16): the forward's "
                                                   "ratio of LDS reads to products",
    }
    if wl.dtype != "bf16":
        roofline.update(bound="latency", peak=None, frac=None)

    result = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded iid Gaussian, resident in HBM)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "head_dim": wl.head_dim,
            "q_len": wl.q_len, "kv_len": wl.kv_len, "num_blocks": wl.num_blocks, "causal": wl.causal,
            "q_idx": wl.q_idx, "path": "host-streamed per-block" if wl.host_streamed else
            ("per-block" if perblock else "fused"),
        },
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "pct_of_probed_peak": (100.0 * value / probed) if probed else None,
        "kernel_ms": kern_ms,
        "kernel_ms_median": sorted(ev_ms)[len(ev_ms) // 2],
        "kernel_ms_min": min(ev_ms),
        "roofline": roofline,
        "outputs_finite": finite,
    }
    result.update(extra)
    if not args.no_cpu_baseline:
        # bound the sample to ~10-30 s of CPU work: every head of the 16-head
        # workloads, every fourth head of the 32-head one
        heads = list(range(wl.heads)) if wl.heads <= 16 else list(range(0, wl.heads, wl.heads // 8))
        base, parity = cpu_baseline(x, wl, o, lse, heads=heads)
        result["cpu_baseline"] = base
        result["parity_sampled"] = parity
    else:
        result["cpu_baseline"] = None
    if not args.no_backward and wl.dtype == "bf16" and not wl.host_streamed:
        heads = [0, wl.heads - 1]
        result["backward"] = backward_measure(x, wl, kb, vb, pos, o, lse, args.bwd_steps, 1, heads)
        if probed:
            result["backward"]["pct_of_probed_peak"] = 100.0 * result["backward"]["value"] / probed
        if probed_rand:
            result["backward"]["pct_of_probed_peak_random_operands"] = (100.0 * result["backward"]["value"] /
                                                                        probed_rand)
        if probed_lds:
            # both backward kernels read about 1 KiB of LDS per product and wave, as the forward does
            result["backward"]["pct_of_probed_peak_random_operands_lds_1k"] = (100.0 * result["backward"]["value"] /
                                                                               probed_lds)
    if not args.no_ffn:
        result["ffn"] = ffn_measure(dev, 10, 2)
        if probed:
            result["ffn"]["pct_of_probed_peak"] = 100.0 * result["ffn"]["value"] / probed
        if probed_rand:
            result["ffn"]["pct_of_probed_peak_random_operands"] = 100.0 * result["ffn"]["value"] / probed_rand
    if not args.no_workloads and args.workload == 3:
        # the timed workload's tensors are no longer needed
        del x, kb, vb, o, lse, ws
        torch.cuda.empty_cache()
        # (the host-streamed pass first: run after the 1M-token workload, its
        # host-to-device copies ran about 50% slower beside the kernels, 78
        # against 57 ms per pass, on every board tried; alone, or after the
        # 32K-chunk workload, it takes the same 57 ms)
        ws_ = {name: workload_summary(dev, cfg) for name, cfg in
               (("chunk32k_p8_host_streamed", 5), ("chunk32k_p8", 2), ("tokens1m_p128", 4))}
        result["workloads"] = {k: ws_[k] for k in ("chunk32k_p8", "tokens1m_p128", "chunk32k_p8_host_streamed")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
