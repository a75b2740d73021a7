"""Host-side checks of the benchmark's work accounting (no GPU)."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from long_context_exact_blockwise_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cfg,pairs", [(1, 262_144), (2, 8_053_080_064), (3, 60_129_607_680),
                                       (4, 8_556_384_256), (5, 8_053_080_064)])
def test_visible_pairs_match_printed_counts(cfg, pairs):
    # the per-head visible-pair counts the baseline table lists for the five workloads
    assert bench.visible_pairs(inputs.CONFIGS[cfg]) == pairs


@pytest.mark.parametrize("q_len,kv_len,p,q_idx,causal", [
    (7, 5, 4, 2, True), (5, 7, 3, 1, True), (8, 8, 4, 0, True), (8, 8, 4, 3, True), (6, 4, 3, 2, False),
    (1, 1, 5, 4, True), (9, 3, 2, 1, True)])
def test_visible_pairs_brute_force(q_len, kv_len, p, q_idx, causal):
    wl = inputs.Workload("t", "bf16", 1, 64, q_len, kv_len, p, causal, q_idx)
    qpos = wl.q_pos0 + np.arange(q_len)
    kpos = np.arange(p * kv_len)
    n = int((kpos[None, :] <= qpos[:, None]).sum()) if causal else q_len * p * kv_len
    assert bench.visible_pairs(wl) == n


def test_flops_config3():
    assert bench.flops(inputs.CONFIGS[3]) == 4 * 16 * 128 * 60_129_607_680


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "ONE GPU" in r.stderr


def test_backward_flops_are_five_products():
    # S, dP, dQ, dK, dV: 2*D flop per visible pair each
    wl = inputs.CONFIGS[3]
    assert bench.bwd_flops(wl) == 10 * 16 * 128 * 60_129_607_680
    assert bench.bwd_flops(wl) * 2 == bench.flops(wl) * 5


def test_committed_counters_give_mfma_busy_and_traffic():
    # the committed summaries match the current kernel source (else both are None)
    busy = bench.read_mfma_busy()
    traffic = bench.read_traffic()
    assert busy is not None and traffic is not None
    assert 0.3 < busy < 1.0
    assert traffic > 5_377_097_728  # at least the algorithmic minimum (Q, K, V once; O, LSE once)


def test_every_profile_summary_matches_the_current_sources():
    # each summary under profiles/ names the hash of the kernel sources and
    # flags it was taken on; a kernel change without new profiles fails here
    want = {"kernel_source_sha256_16": bench.kernel_hash(),
            "backward_source_and_flags_sha256_16": bench.backward_hash(),
            "feedforward_source_and_flags_sha256_16": bench.feedforward_hash()}
    prof = os.path.join(ROOT, "profiles")
    seen = 0
    for name in sorted(os.listdir(prof)):
        for line in open(os.path.join(prof, name)):
            key = line.split(":", 1)[0].strip()
            if key in want:
                assert line.split(":", 1)[1].strip() == want[key], (name, key)
                seen += 1
    assert seen >= 8
