"""The blockwise-feedforward oracle against its pins, and plausible mistakes
planted in a copy of it (each must be caught by at least one pin)."""

import os
import types

import pytest

from oracle import ffn as ffn_oracle
from tests import _pins_ffn

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ffn.py")


@pytest.mark.parametrize("pin", _pins_ffn.ALL_FFN_PINS, ids=lambda f: f.__name__)
def test_ffn_pin(pin):
    pin(ffn_oracle)


MUTANTS = {
    "cubic_coefficient": ("0.044715 * x ** 3", "0.0447 * x ** 3"),
    "sqrt_two_over_pi": ("np.sqrt(2.0 / np.pi) * (x", "np.sqrt(2.0) / np.pi * (x"),
    "half_missing": ("return 0.5 * x * (1.0 + np.tanh", "return x * (1.0 + np.tanh"),
    "no_b1": ("h = gelu_tanh(x[r0:r0 + step] @ w1.T + b1)", "h = gelu_tanh(x[r0:r0 + step] @ w1.T)"),
    "no_b2": ("y[r0:r0 + step] = h @ w2.T + b2", "y[r0:r0 + step] = h @ w2.T"),
    "act_after_second": ("y[r0:r0 + step] = h @ w2.T + b2", "y[r0:r0 + step] = gelu_tanh(h @ w2.T + b2)"),
    "w1_untransposed": ("x[r0:r0 + step] @ w1.T + b1", "x[r0:r0 + step] @ w2 + b1"),
    "block_gap": ("for r0 in range(0, n, max(step, 1)):", "for r0 in range(0, n, max(step, 1) + 1):"),
}


def _mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    mod = types.ModuleType(f"ffn_mutant_{name}")
    exec(compile(src.replace(old, new), f"<ffn mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_ffn_planted_mistake_is_caught(name):
    mod = _mutant(name, *MUTANTS[name])
    caught = []
    for pin in _pins_ffn.ALL_FFN_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects the planted mistake {name}"
