"""The backward oracle against its pins, and plausible mistakes planted in a
copy of it (each must be caught by at least one pin)."""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as fwd_oracle
from oracle import backward as bwd_oracle
from tests import _pins_bwd

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "backward.py")


@pytest.mark.parametrize("pin", _pins_bwd.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin(bwd_oracle, fwd_oracle)


def test_bwd_empty_inputs():
    q = np.zeros((1, 0, 1, 4))
    dq, dk, dv = oracle.ring_attention_bwd(q, [np.zeros((1, 3, 1, 4))], [np.zeros((1, 3, 1, 4))], 0, [0], True, q)
    assert dq.shape == q.shape and dk[0].shape == (1, 3, 1, 4) and not dk[0].any() and not dv[0].any()


MUTANTS = {
    "no_delta": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "dq_no_scale": ("dq[b, :, h, :] = scale * (ds @ kh)", "dq[b, :, h, :] = ds @ kh"),
    "dk_sign": ("dkh = scale * (ds.T @ qh)", "dkh = -scale * (ds.T @ qh)"),
    "dp_wrong_operand": ("dp = doh @ vh.T", "dp = doh @ kh.T"),
    "mask_ignored": ("s = np.where(vis, scale * (qh @ kh.T), -np.inf)", "s = scale * (qh @ kh.T)"),
    "dv_from_ds": ("dvh = p.T @ doh", "dvh = ds.T @ doh"),
    "blocks_in_given_order": ("for pos, j in enumerate(order):", "for pos, j in enumerate(range(nblk)):"),
    # the chosen-keys gradient (key_rows_bwd)
    "key_rows_delta_over_chosen": ("delta_r = (p * dp).sum(axis=1, keepdims=True)",
                                   "delta_r = (p[:, sel] * dp[:, sel]).sum(axis=1, keepdims=True)"),
    "key_rows_normaliser_over_chosen": ("p = e / e.sum(axis=1, keepdims=True)",
                                        "p = e / e[:, sel].sum(axis=1, keepdims=True)"),
    "key_rows_chunk_positions": ("vis = visible(q_pos[r0:r1], kv_pos, causal)",
                                 "vis = visible(q_pos[:r1 - r0], kv_pos, causal)"),
    "key_rows_block_offset": ("sel = np.array([starts[j] + i for j, i in key_rows]",
                              "sel = np.array([i for j, i in key_rows]"),
    "key_rows_dk_no_scale": ("dk[b, :, h, :] += scale * (ds_sel.T @ qc)", "dk[b, :, h, :] += ds_sel.T @ qc"),
}


def _mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"bwd_mutant_{name}")
    exec(compile(src, f"<bwd mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_planted_mistake_is_caught(name):
    mod = _mutant(name, *MUTANTS[name])
    caught = []
    for pin in _pins_bwd.ALL_BWD_PINS:
        try:
            pin(mod, fwd_oracle)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects the planted mistake {name}"
