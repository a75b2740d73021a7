"""Plausible mistakes planted in a copy of the oracle (on the CPU) must each be
caught by at least one pin: evidence that the pins are strong enough."""

import importlib.util
import os
import sys
import types

import pytest

from tests import _pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "scale_1_over_d": ("1.0 / math.sqrt(head_dim)", "1.0 / head_dim"),
    "mask_strict": ("kv_pos[None, :] <= q_pos[:, None]", "kv_pos[None, :] < q_pos[:, None]"),
    "mask_reversed": ("kv_pos[None, :] <= q_pos[:, None]", "kv_pos[None, :] >= q_pos[:, None]"),
    "exp_sign": ("e = np.exp(s - m)  #", "e = np.exp(m - s)  #"),
    "lse_drops_max": ("lse[has] = m[:, 0] + np.log(l[:, 0])", "lse[has] = np.log(l[:, 0])"),
    "wrong_operand": ("out[has] = (e @ v) / l", "out[has] = (e @ k[:, :v.shape[1]]) / l"),
    "no_normalise": ("out[has] = (e @ v) / l", "out[has] = (e @ v)"),
    "block_positions": ("ps.append(int(kv_pos0s[j])", "ps.append(int(kv_pos0s[0])"),
    "local_positions": ("q_pos = int(q_pos0) + int(pos_stride) * rows", "q_pos = int(pos_stride) * rows"),
    "state_normalised": ("acc[b, h, has, :] = e @ vh", "acc[b, h, has, :] = (e @ vh) / e.sum(axis=1)[:, None]"),
    "state_log2": ("m[b, h, has] = mh", "m[b, h, has] = mh / 0.6931471805599453"),
    "stride_kv_ignored": ("int(pos_stride) * np.arange(kb.shape[1]", "np.arange(kb.shape[1]"),
    "stride_q_ignored": ("q_pos = int(q_pos0) + int(pos_stride) * rows", "q_pos = int(q_pos0) + rows"),
    "state_stride_ignored": ("visible(int(q_pos0) + int(pos_stride) * np.arange(sq)",
                             "visible(int(q_pos0) + np.arange(sq)"),
}


def _load_mutant(name, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _load_mutant(name, *MUTANTS[name])
    caught = []
    for pin in _pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects the planted mistake {name}"
