"""Host checks of the build's job list: every source is compiled, the backward
source as two objects (one kernel each) with its own scheduling strategy, and the
scheduler flag that the fused kernel's traffic counters are tied to is part of
the hash that bench.py checks."""

from __future__ import annotations

import os

from long_context_exact_blockwise_amd import build


def test_every_source_compiled_once_or_split():
    jobs = list(build._jobs())
    srcs = {s for s, _, _ in jobs}
    assert srcs == set(build.SOURCES)
    names = [n for _, n, _ in jobs]
    assert len(names) == len(set(names)), "object names must be unique"
    for s in build.SOURCES:
        assert os.path.exists(os.path.join(build.CSRC, s))


def test_backward_split_into_dq_and_dkdv_objects():
    bwd = {n: f for s, n, f in build._jobs() if s == "attn_bwd.hip"}
    assert set(bwd) == {"attn_bwd_dq", "attn_bwd_dkdv"}
    assert "-DRA_BWD_PART=1" in bwd["attn_bwd_dq"] and "-DRA_BWD_PART=2" in bwd["attn_bwd_dkdv"]
    ilp = "-amdgpu-sched-strategy=iterative-ilp"
    max_ilp = "-amdgpu-sched-strategy=max-ilp"
    assert ilp not in bwd["attn_bwd_dq"] and ilp in bwd["attn_bwd_dkdv"]
    assert max_ilp in bwd["attn_bwd_dq"] and max_ilp not in bwd["attn_bwd_dkdv"]


def test_forward_flags_in_traffic_hash(monkeypatch):
    import bench
    h0 = bench.kernel_hash()
    monkeypatch.setitem(build.SOURCE_FLAGS, "attn_bf16.hip", [])
    assert bench.kernel_hash() != h0


def test_checking_library_differs_only_in_the_host_layer():
    jobs = {n: (s, f) for s, n, f in build._jobs()}
    assert jobs["ringattn_api_check"] == ("ringattn_api.hip", ["-DRA_POISON_STAGING=1"])
    assert jobs["ringattn_api"] == ("ringattn_api.hip", [])
    assert build.CHECK_ONLY == {"ringattn_api_check"} and build.MAIN_ONLY == {"ringattn_api"}
