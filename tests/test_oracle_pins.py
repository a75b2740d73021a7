"""The fp64 oracle against facts other than itself (brute force, closed forms,
invariants, a library routine, hand-derived worked examples)."""

import numpy as np
import pytest

import oracle
from tests import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attention)


def test_empty_inputs():
    q = np.zeros((1, 0, 2, 4))
    o, lse = oracle.ring_attention(q, [], [], 0, [], True)
    assert o.shape == (1, 0, 2, 4) and lse.shape == (1, 2, 0)
    q = np.ones((1, 3, 2, 4))
    o, lse = oracle.ring_attention(q, [], [], 0, [], False)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    m, l, acc = oracle.partial_state(q, [], [], 0, [], False)
    assert np.all(m == -np.inf) and np.all(l == 0) and np.all(acc == 0)


def test_sampled_rows_match_full():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 9, 2, 8))
    kb = [rng.standard_normal((1, 5, 2, 8)) for _ in range(3)]
    vb = [rng.standard_normal((1, 5, 2, 8)) for _ in range(3)]
    o, lse = oracle.ring_attention(q, kb, vb, 6, [0, 5, 10], True)
    rows = [0, 4, 8]
    o2, lse2 = oracle.ring_attention(q, kb, vb, 6, [0, 5, 10], True, rows=rows, heads=[1])
    assert np.array_equal(o2[:, :, 0], o[:, rows, 1]) and np.array_equal(lse2[:, 0], lse[:, 1, rows])
