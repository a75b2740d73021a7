"""Checks that pin the fp64 blockwise-feedforward oracle to facts other than
itself.  Each takes the oracle module so the same checks can run against
copies with a planted mistake."""

from __future__ import annotations

import math

import numpy as np
import torch


def _case(seed, n=37, d=8, f=32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    w1 = rng.standard_normal((f, d)) / math.sqrt(d)
    b1 = 0.3 * rng.standard_normal(f)
    w2 = rng.standard_normal((d, f)) / math.sqrt(f)
    b2 = 0.3 * rng.standard_normal(d)
    return x, w1, b1, w2, b2


def pin_gelu_library(ffn):
    """torch's GELU with approximate='tanh' in fp64: an independent
    implementation of the same published formula."""
    x = np.linspace(-8.0, 8.0, 1601)
    ref = torch.nn.functional.gelu(torch.tensor(x), approximate="tanh").numpy()
    assert np.allclose(ffn.gelu_tanh(x), ref, rtol=0, atol=1e-15)


def pin_gelu_closed_forms(ffn):
    """gelu(0) = 0; gelu(x) - gelu(-x) = x (the tanh argument is odd);
    gelu(x) -> x for large x and -> 0 for very negative x; and within 2e-3
    of the erf form x Phi(x) everywhere (the tanh form approximates it)."""
    x = np.linspace(-6.0, 6.0, 1201)
    g = ffn.gelu_tanh(x)
    assert ffn.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(g - ffn.gelu_tanh(-x), x, rtol=0, atol=1e-14)
    assert abs(ffn.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(ffn.gelu_tanh(np.array([-30.0]))[0]) < 1e-12
    erf_form = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    assert np.max(np.abs(g - erf_form)) < 2e-3


def pin_ffn_torch_modules(ffn):
    """torch.nn.Linear -> GELU(tanh) -> Linear in fp64 with the same weights."""
    x, w1, b1, w2, b2 = _case(1)
    l1 = torch.nn.Linear(w1.shape[1], w1.shape[0]).double()
    l2 = torch.nn.Linear(w2.shape[1], w2.shape[0]).double()
    with torch.no_grad():
        l1.weight.copy_(torch.tensor(w1))
        l1.bias.copy_(torch.tensor(b1))
        l2.weight.copy_(torch.tensor(w2))
        l2.bias.copy_(torch.tensor(b2))
        ref = l2(torch.nn.GELU(approximate="tanh")(l1(torch.tensor(x)))).numpy()
    assert np.allclose(ffn.blockwise_ffn(x, w1, b1, w2, b2), ref, rtol=0, atol=1e-13)


def pin_ffn_closed_forms(ffn):
    """F = d, W1 = W2 = I, zero biases: y = gelu(x).  A constant c added to
    b2 adds c to every output.  With W1 = 0 every row is gelu(b1) W2^T + b2."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 6))
    eye = np.eye(6)
    z = np.zeros(6)
    assert np.allclose(ffn.blockwise_ffn(x, eye, z, eye, z), ffn.gelu_tanh(x), rtol=0, atol=1e-15)
    x, w1, b1, w2, b2 = _case(3)
    y = ffn.blockwise_ffn(x, w1, b1, w2, b2)
    assert np.allclose(ffn.blockwise_ffn(x, w1, b1, w2, b2 + 1.25), y + 1.25, rtol=0, atol=1e-13)
    y0 = ffn.blockwise_ffn(x, np.zeros_like(w1), b1, w2, b2)
    expect = w2 @ (0.5 * b1 * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (b1 + 0.044715 * b1 ** 3)))) + b2
    assert np.allclose(y0, np.broadcast_to(expect, y0.shape), rtol=0, atol=1e-13)


def pin_ffn_blockwise_equals_whole(ffn):
    """Row blocks of any size (dividing N or not) give the whole-chunk
    result (to fp64 rounding: BLAS may sum in another order for another
    shape): the network is position-wise."""
    x, w1, b1, w2, b2 = _case(4)
    whole = ffn.blockwise_ffn(x, w1, b1, w2, b2)
    for r in (1, 5, 16, 37, 100):
        assert np.allclose(ffn.blockwise_ffn(x, w1, b1, w2, b2, block_rows=r), whole, rtol=0, atol=1e-14)
    # and row i depends on x_i alone
    x2 = x.copy()
    x2[3] += 1.0
    y2 = ffn.blockwise_ffn(x2, w1, b1, w2, b2)
    assert np.allclose(np.delete(y2, 3, axis=0), np.delete(whole, 3, axis=0), rtol=0, atol=1e-14)
    assert not np.allclose(y2[3], whole[3])


ALL_FFN_PINS = [pin_gelu_library, pin_gelu_closed_forms, pin_ffn_torch_modules, pin_ffn_closed_forms,
                pin_ffn_blockwise_equals_whole]
