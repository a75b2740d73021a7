"""Race checks of the host-streamed ring pass (two staging slots, a copy stream
and per-slot events), run through the checking build of the library, which
fills every slot region with NaN on the copy stream just before each copy
into it.  If a kernel read a slot before its copy had landed, or a copy
overwrote a slot that kernels of the block two steps back were still
reading, the NaN (or the wrong block) would reach the output.  Each case
must be bitwise equal to the device-resident per-block pass and match the
fp64 oracle.  This is the bug of "The Synchronous Send/Recv Trap" in "Ring
Attention: Train 1M Tokens on 8GB GPUs in 2026": garbage K/V states when the
compute does not wait for the transfer.

Many small blocks make each slot be reused many times (16 times per slot for
32 blocks)."""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra
from tests._gpu_common import compare, cuda, gpu_rows, oracle_ref
from tests.test_gpu_varlen_striped import _oracle_varlen, _poison_padding

pytestmark = pytest.mark.gpu

CHECK_LIB = os.path.join(os.path.dirname(ra.LIB_PATH), "libringattn_check.so")


@pytest.fixture
def checking_library(monkeypatch):
    lib = ra.load(CHECK_LIB)
    monkeypatch.setattr(ra, "_lib", lib)
    return lib


def _streamed(x, order, valid=None, causal=True):
    wl = x.wl
    vo = None if valid is None else [valid[j] for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    hk = [x.k_block(j).contiguous().cpu().pin_memory() for j in order]
    hv = [x.v_block(j).contiguous().cpu().pin_memory() for j in order]
    desc = ra.make_desc(x.q, hk[0], q_pos0=wl.q_pos0, causal=causal)
    m, l, acc = ra.state_buffers(desc, x.q.device)
    stage_k = [torch.empty(hk[0].shape, dtype=hk[0].dtype, device=x.q.device) for _ in range(2)]
    stage_v = [torch.empty(hv[0].shape, dtype=hv[0].dtype, device=x.q.device) for _ in range(2)]
    o = torch.empty_like(x.q)
    lse = torch.empty((wl.batch, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
    ra.ringattn_ring_fwd(desc, x.q, hk, hv, pos, o, lse, m, l, acc, kv_valid=vo, kv_on_host=True, stage_k=stage_k,
                         stage_v=stage_v, copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    return o, lse


def _resident(x, order, valid=None, causal=True):
    wl = x.wl
    vo = None if valid is None else [valid[j] for j in order]
    o, lse = ra.ring_forward(x.q, [x.k_block(j) for j in order], [x.v_block(j) for j in order],
                             [wl.kv_pos0(j) for j in order], q_pos0=wl.q_pos0, causal=causal, perblock=True,
                             kv_valid=vo)
    torch.cuda.synchronize()
    return o, lse


def test_many_blocks_slot_reuse(checking_library):
    """32 blocks of 256 keys, causal, last device of the ring: each slot is
    refilled 16 times."""
    p = 32
    wl = inputs.Workload("race P32x256 causal", "bf16", 2, 128, 256, 256, p, True, p - 1)
    print(f"streamed race: {wl.name}", flush=True)
    x = inputs.make_inputs(wl, cuda(), seed=91)
    order = ra.ringattn_ring_order(p - 1, p)
    o, lse = _streamed(x, order)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, l_ref = _resident(x, order)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    ref_o, ref_l = oracle_ref(x)
    print(compare(*gpu_rows(o, lse), ref_o, ref_l, "bf16", wl.name))


def test_many_ragged_blocks_batch2_noncausal(checking_library):
    """24 blocks of unequal valid length (1..200 keys of 200, NaN padding),
    batch 2 (2-D copies), non-causal: slot regions of different sizes."""
    p, ck = 24, 200
    wl = inputs.Workload("race P24x200 ragged B2 noncausal", "bf16", 2, 128, 192, ck, p, False, 0, batch=2)
    print(f"streamed race: {wl.name}", flush=True)
    x = inputs.make_inputs(wl, cuda(), seed=92)
    valid = [int(v) for v in np.random.default_rng(93).integers(1, ck + 1, size=p)]
    _poison_padding(x, valid)
    order = list(np.random.default_rng(94).permutation(p))
    o, lse = _streamed(x, order, valid=valid, causal=False)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, l_ref = _resident(x, order, valid=valid, causal=False)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    ref_o, ref_l = _oracle_varlen(x, valid)
    print(compare(*gpu_rows(o, lse), ref_o, ref_l, "bf16", wl.name))


def test_host_streamed_workload_poisoned(checking_library):
    """The host-streamed workload at full size (16 heads, 32768 rows, 8 blocks
    of 32768 keys from pinned host memory, causal, last device), through the
    checking build: bitwise equal to the device-resident per-block pass."""
    wl = inputs.CONFIGS[5]
    print(f"streamed race: {wl.name}", flush=True)
    x = inputs.make_inputs(wl, cuda(), seed=0)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    o, lse = _streamed(x, order)
    o_ref, l_ref = _resident(x, order)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
