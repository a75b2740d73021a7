"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Sizes span several tiles with ragged tails (Q tiles of 128 rows, K tiles of
64 keys for bf16; 64 rows / 16 keys for fp32) and cover every block class."""

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra
from tests._gpu_common import compare, cuda, gpu_rows, lse_natural_from_state, oracle_ref, run_hip, small

pytestmark = pytest.mark.gpu


def _check(x, order=None, perblock=False, out_dtype=None, what=""):
    o, lse = run_hip(x, order=order, perblock=perblock, out_dtype=out_dtype)
    ref_o, ref_l = oracle_ref(x)
    go, gl = gpu_rows(o, lse)
    return compare(go, gl, ref_o, ref_l, x.wl.dtype, what or x.wl.name)


@pytest.mark.parametrize("perblock", [False, True], ids=["fused", "perblock"])
def test_config1_fp32(perblock):
    x = inputs.make_inputs(inputs.CONFIGS[1], cuda(), seed=0)
    err = _check(x, perblock=perblock)
    print("config1", perblock, err)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("perblock", [False, True], ids=["fused", "perblock"])
def test_bf16_ragged(d, causal, perblock):
    wl = small(d=d, causal=causal)
    x = inputs.make_inputs(wl, cuda(), seed=3)
    print(_check(x, perblock=perblock))


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_ragged_causal(d):
    wl = small(dtype="f32", d=d, q_len=150, kv_len=70, p=3, q_idx=1)
    x = inputs.make_inputs(wl, cuda(), seed=4)
    print(_check(x))
    print(_check(x, perblock=True))


def test_bf16_out_fp32():
    x = inputs.make_inputs(small(), cuda(), seed=5)
    print(_check(x, out_dtype=torch.float32))


@pytest.mark.parametrize("q_idx", [0, 1, 2, 3])
def test_q_idx_sweep_ring_order(q_idx):
    """One device's share for every device of a 4-ring: skipped, full and
    diagonal blocks, processed in ring order (q_idx - s) mod P."""
    wl = small(heads=2, d=128, q_len=256, kv_len=256, p=4, q_idx=q_idx)
    x = inputs.make_inputs(wl, cuda(), seed=10 + q_idx)
    order = ra.ringattn_ring_order(q_idx, 4)
    print(_check(x, order=order))
    print(_check(x, order=order, perblock=True))


def test_peaked_softmax():
    """Q multiplied by 8: scores with std ~4, |O| of order 0.1-1, so the bf16
    gate is meaningful."""
    wl = small(q_len=384, kv_len=256, p=3, q_idx=2)
    x = inputs.make_inputs(wl, cuda(), seed=6, q_mult=8.0)
    print(_check(x, order=[2, 1, 0]))


def test_late_max_jump():
    """The block processed last has its keys multiplied by 4: the running max
    moves late and the carried state is rescaled by factors << 1."""
    wl = small(q_len=256, kv_len=256, p=4, q_idx=3)
    order = ra.ringattn_ring_order(3, 4)
    x = inputs.make_inputs(wl, cuda(), seed=7, k_block_mult={order[-1]: 4.0})
    print(_check(x, order=order))
    print(_check(x, order=order, perblock=True))


def test_block_order_does_not_matter():
    wl = small(q_len=128, kv_len=128, p=5, q_idx=4)
    x = inputs.make_inputs(wl, cuda(), seed=8)
    outs = []
    for order in ([4, 3, 2, 1, 0], [0, 1, 2, 3, 4], [2, 4, 0, 3, 1]):
        _check(x, order=order)
        outs.append(run_hip(x, order=order))
    for o, l in outs[1:]:
        assert torch.allclose(o.float(), outs[0][0].float(), atol=2e-2, rtol=0)
        assert torch.allclose(l, outs[0][1], atol=1e-3, rtol=1e-4)


@pytest.mark.parametrize("causal,valid", [(True, None), (False, None), (True, (2048, 1999, 2048, 1037))],
                         ids=["causal", "noncausal", "causal_ragged"])
def test_long_tile_runs(causal, valid):
    """2048 rows against 4 blocks of 2048 keys (32 tiles each, K and V in
    separate allocations), in ring order: most tiles run in long stretches
    with no cursor test, broken by block ends, ragged last tiles and the
    causal diagonal."""
    wl = small(q_len=2048, kv_len=2048, p=4, causal=causal, q_idx=3)
    x = inputs.make_inputs(wl, cuda(), seed=12)
    order = ra.ringattn_ring_order(3, 4)
    if valid is None:
        print(_check(x, order=order))
        return
    from tests.test_gpu_varlen_striped import _oracle_varlen, _poison_padding
    _poison_padding(x, valid)
    o, lse = ra.ring_forward(x.q, [x.k_block(j) for j in order], [x.v_block(j) for j in order],
                             [wl.kv_pos0(j) for j in order], q_pos0=wl.q_pos0, causal=causal,
                             kv_valid=[valid[j] for j in order])
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle_varlen(x, list(valid))
    print(compare(*gpu_rows(o, lse), ref_o, ref_l, "bf16", "long tile runs, ragged"))


def test_fused_matches_perblock():
    x = inputs.make_inputs(small(q_len=512, kv_len=320, p=3, q_idx=1), cuda(), seed=9)
    o1, l1 = run_hip(x)
    o2, l2 = run_hip(x, perblock=True)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4 * max(1.0, l1.abs().max().item())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_after_each_block(dtype):
    """init_state, then block_fwd one block at a time: after k blocks the state
    represents the attention over those k blocks (acc/l and m + ln l)."""
    wl = small(dtype=dtype, q_len=200, kv_len=160, p=3, q_idx=1)
    x = inputs.make_inputs(wl, cuda(), seed=11)
    order = ra.ringattn_ring_order(1, 3)
    desc = ra.make_desc(x.q, x.k_block(0), q_pos0=wl.q_pos0, causal=True)
    m, l, acc = ra.state_buffers(desc, x.q.device)
    ra.ringattn_init_state(desc, m, l, acc)
    q64 = inputs.to_f64(x.q)
    for k in range(1, 4):
        j = order[k - 1]
        ra.ringattn_block_fwd(desc, x.q, x.k_block(j), x.v_block(j), wl.kv_pos0(j), m, l, acc)
        torch.cuda.synchronize()
        seen = order[:k]
        om, ol, oacc = oracle.partial_state(q64, [inputs.to_f64(x.k_block(j)) for j in seen],
                                            [inputs.to_f64(x.v_block(j)) for j in seen], wl.q_pos0,
                                            [wl.kv_pos0(j) for j in seen], True)
        gm, gl, gacc = (t.double().cpu().numpy() for t in (m, l, acc))
        fin = ol > 0
        assert np.array_equal(gl > 0, fin)
        with np.errstate(invalid="ignore", divide="ignore"):
            o_gpu = np.where(fin[..., None], gacc / np.where(fin, gl, 1)[..., None], 0)
            o_ref = np.where(fin[..., None], oacc / np.where(fin, ol, 1)[..., None], 0)
        # state layout [B, H, Sq, D] -> compare as [B, Sq, H, D]
        compare(np.transpose(o_gpu, (0, 2, 1, 3)), lse_natural_from_state(gm, gl),
                np.transpose(o_ref, (0, 2, 1, 3)), lse_natural_from_state(om, ol), dtype, f"after {k} blocks")
    o = torch.empty_like(x.q)
    lse = torch.empty((1, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
    ra.ringattn_finalize(desc, m, l, acc, o, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_ref(x)
    compare(*gpu_rows(o, lse), ref_o, ref_l, dtype, "finalized")


def test_state_checkpoint_roundtrip_is_bitwise():
    """Stop after one block, move the state to the host and back, continue:
    identical bits to an uninterrupted per-block pass."""
    wl = small(q_len=256, kv_len=192, p=3, q_idx=2)
    x = inputs.make_inputs(wl, cuda(), seed=12)
    desc = ra.make_desc(x.q, x.k_block(0), q_pos0=wl.q_pos0, causal=True)

    def run(interrupt):
        m, l, acc = ra.state_buffers(desc, x.q.device)
        ra.ringattn_init_state(desc, m, l, acc)
        for i, j in enumerate([2, 1, 0]):
            ra.ringattn_block_fwd(desc, x.q, x.k_block(j), x.v_block(j), wl.kv_pos0(j), m, l, acc)
            if interrupt and i == 0:
                host = [t.cpu() for t in (m, l, acc)]
                m, l, acc = (t.to(x.q.device) for t in host)
        o = torch.empty_like(x.q)
        lse = torch.empty((1, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
        ra.ringattn_finalize(desc, m, l, acc, o, lse)
        torch.cuda.synchronize()
        return o, lse

    o1, l1 = run(False)
    o2, l2 = run(True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_and_degenerate():
    dev = cuda()
    # no blocks: every row sees nothing -> O = 0, LSE = -inf
    q = torch.randn(1, 130, 2, 128, device=dev).bfloat16()
    o, lse = ra.ring_forward(q, [], [], [], q_pos0=0, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # causal, every block after the chunk: all skipped
    k = torch.randn(1, 64, 2, 128, device=dev).bfloat16()
    o, lse = ra.ring_forward(q, [k, k], [k, k], [500, 1000], q_pos0=0, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # empty query chunk: nothing to do
    q0 = torch.empty(1, 0, 2, 128, device=dev, dtype=torch.bfloat16)
    o0, l0 = ra.ring_forward(q0, [k], [k], [0], q_pos0=0, causal=False)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and l0.numel() == 0
    # first global row sees exactly its own key: O = v_0 (rounded to bf16)
    kv = torch.randn(1, 64, 2, 128, device=dev).bfloat16()
    o, lse = ra.ring_forward(q[:, :64], [kv], [kv], [0], q_pos0=0, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[0, 0], kv[0, 0])
    # a single key per row, one-key blocks of length 1 (ragged everywhere)
    k1 = torch.randn(1, 1, 2, 128, device=dev).bfloat16()
    v1 = torch.randn(1, 1, 2, 128, device=dev).bfloat16()
    o, lse = ra.ring_forward(q[:, :3], [k1], [v1], [0], q_pos0=5, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, v1.expand(1, 3, 2, 128))


def test_long_ring_segments():
    """More blocks than one fused launch carries: the state crosses launches
    through the workspace."""
    wl = small(heads=1, d=128, q_len=128, kv_len=64, p=70, q_idx=0, causal=False)
    x = inputs.make_inputs(wl, cuda(), seed=13)
    print(_check(x))
    wl2 = inputs.Workload("causal long", "bf16", 1, 128, 64, 64, 70, True, 69)
    x2 = inputs.make_inputs(wl2, cuda(), seed=14)
    print(_check(x2, order=ra.ringattn_ring_order(69, 70)))


def test_host_streamed_equals_perblock_bitwise():
    wl = small(heads=2, q_len=256, kv_len=256, p=4, q_idx=3)
    x = inputs.make_inputs(wl, cuda(), seed=15)
    order = ra.ringattn_ring_order(3, 4)
    o_ref, l_ref = run_hip(x, order=order, perblock=True)
    hk = [x.k_block(j).cpu().pin_memory() for j in order]
    hv = [x.v_block(j).cpu().pin_memory() for j in order]
    desc = ra.make_desc(x.q, hk[0], q_pos0=wl.q_pos0, causal=True)
    m, l, acc = ra.state_buffers(desc, x.q.device)
    stage_k = [torch.empty_like(x.k_block(0)).contiguous() for _ in range(2)]
    stage_v = [torch.empty_like(x.v_block(0)).contiguous() for _ in range(2)]
    o = torch.empty_like(x.q)
    lse = torch.empty((1, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
    copy = torch.cuda.Stream()
    ra.ringattn_ring_fwd(desc, x.q, hk, hv, [wl.kv_pos0(j) for j in order], o, lse, m, l, acc, kv_on_host=True,
                         stage_k=stage_k, stage_v=stage_v, copy_stream=copy)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_pageable_host_blocks_rejected():
    wl = small(heads=2, q_len=128, kv_len=128, p=2, q_idx=1)
    x = inputs.make_inputs(wl, cuda(), seed=16)
    hk = [x.k_block(j).cpu() for j in range(2)]  # pageable
    desc = ra.make_desc(x.q, hk[0], q_pos0=wl.q_pos0, causal=True)
    m, l, acc = ra.state_buffers(desc, x.q.device)
    st = [torch.empty_like(x.k_block(0)).contiguous() for _ in range(2)]
    o = torch.empty_like(x.q)
    lse = torch.empty((1, 2, 128), dtype=torch.float32, device=x.q.device)
    with pytest.raises(ra.RingAttnError) as e:
        ra.ringattn_ring_fwd(desc, x.q, hk, hk, [0, 128], o, lse, m, l, acc, kv_on_host=True, stage_k=st,
                             stage_v=st, copy_stream=torch.cuda.Stream())
    assert e.value.status == ra.RA_E_MEMTYPE
    assert torch.isfinite(x.q.float()).all()
