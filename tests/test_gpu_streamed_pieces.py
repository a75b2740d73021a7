"""GPU parity for the per-block ring pass, which processes the first two
visible blocks in pieces of whole 64-key tiles: host-streamed blocks (batch 2
through 2-D copies, ragged valid lengths whose last piece is not a whole tile,
padding poisoned with NaN) against the device-resident per-block pass
(bitwise) and against the fp64 oracle."""

from __future__ import annotations

import pytest
import torch

from long_context_exact_blockwise_amd import inputs
from long_context_exact_blockwise_amd import ringattn as ra
from tests._gpu_common import compare, cuda, gpu_rows
from tests.test_gpu_varlen_striped import _oracle_varlen, _poison_padding

pytestmark = pytest.mark.gpu

VALID = [1000, 777, 1000]  # block 1: pieces of 256 rows, the last one 9 rows


@pytest.mark.parametrize("batch,causal", [(2, True), (2, False), (1, True)])
def test_streamed_pieces_match_resident_and_oracle(batch, causal):
    wl = inputs.Workload(f"pieces B{batch}", "bf16", 2, 128, 300, 1000, 3, causal, 2, batch=batch)
    print(f"streamed pieces: batch {batch} causal {causal}", flush=True)
    x = inputs.make_inputs(wl, cuda(), seed=40 + batch)
    _poison_padding(x, VALID)
    order = ra.ringattn_ring_order(wl.q_idx, wl.num_blocks)
    vo = [VALID[j] for j in order]
    pos = [wl.kv_pos0(j) for j in order]
    o_ref, l_ref = ra.ring_forward(x.q, [x.k_block(j) for j in order], [x.v_block(j) for j in order], pos,
                                   q_pos0=wl.q_pos0, causal=causal, perblock=True, kv_valid=vo)
    hk = [x.k_block(j).contiguous().cpu().pin_memory() for j in order]
    hv = [x.v_block(j).contiguous().cpu().pin_memory() for j in order]
    desc = ra.make_desc(x.q, hk[0], q_pos0=wl.q_pos0, causal=causal)
    m, l, acc = ra.state_buffers(desc, x.q.device)
    stage_k = [torch.empty(hk[0].shape, dtype=hk[0].dtype, device=x.q.device) for _ in range(2)]
    stage_v = [torch.empty(hv[0].shape, dtype=hv[0].dtype, device=x.q.device) for _ in range(2)]
    o = torch.empty_like(x.q)
    lse = torch.empty((batch, wl.heads, wl.q_len), dtype=torch.float32, device=x.q.device)
    ra.ringattn_ring_fwd(desc, x.q, hk, hv, pos, o, lse, m, l, acc, kv_valid=vo, kv_on_host=True, stage_k=stage_k,
                         stage_v=stage_v, copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    ref_o, ref_l = _oracle_varlen(x, VALID)
    print(compare(*gpu_rows(o, lse), ref_o, ref_l, "bf16", f"streamed pieces B{batch} causal={causal}"))
