"""Pins for the oracle's epilogue, act(ref + bias[j]) in FP64 (CPU only).

The template article names bias add, ReLU and GELU as what an epilogue
inserts before the result is written back (§2.3, §6). GELU is taken in its
exact form y * Phi(y) = 0.5 * y * (1 + erf(y / sqrt 2)).

Pinned by: a Taylor series of erf summed independently in Python, the
identity GELU(y) - GELU(-y) = y, the limits GELU(y) = y and GELU(-y) = 0 for
large y, GELU(0) = 0, ReLU and the bias by definition, and column indexing
against an explicit loop.
"""

import math

import numpy as np
import pytest

import oracle


def _gelu_series(y: float) -> float:
    """0.5*y*(1 + erf(y/sqrt2)) with erf from its Maclaurin series (|y| <= 3)."""
    z = y / math.sqrt(2.0)
    term, total, n = z, z, 0
    while abs(term) > 1e-19 * max(1.0, abs(total)):
        n += 1
        term *= -z * z / n
        total += term / (2 * n + 1)
    erf = 2.0 / math.sqrt(math.pi) * total
    return 0.5 * y * (1.0 + erf)


def test_gelu_matches_series():
    ys = np.linspace(-3.0, 3.0, 601)
    got = oracle.epilogue(ys[None, :], act=oracle.ACT_GELU)[0]
    want = np.array([_gelu_series(float(y)) for y in ys])
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


def test_gelu_identities_and_limits():
    ys = np.concatenate([np.linspace(-20, 20, 4001), [1e-300, 1e300]])
    pos = oracle.epilogue(ys[None, :], act=oracle.ACT_GELU)[0]
    neg = oracle.epilogue(-ys[None, :], act=oracle.ACT_GELU)[0]
    finite = np.abs(ys) < 1e200
    assert np.allclose((pos - neg)[finite], ys[finite], rtol=1e-15, atol=1e-300)
    big = ys >= 10.0
    assert np.array_equal(pos[big], ys[big]) and np.all(np.abs(neg[big]) < 1e-20)
    assert oracle.epilogue(np.zeros((1, 1)), act=oracle.ACT_GELU)[0, 0] == 0.0


def test_relu_and_bias_by_definition():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((7, 9))
    bias = rng.standard_normal(20).astype(np.float32)
    cols = np.array([0, 3, 19, 4, 4, 11, 2, 8, 15])
    got_none = oracle.epilogue(ref, bias, oracle.ACT_NONE, cols)
    got_relu = oracle.epilogue(ref, bias, oracle.ACT_RELU, cols)
    for r in range(7):
        for c in range(9):
            y = ref[r, c] + float(bias[cols[c]])
            assert got_none[r, c] == y
            assert got_relu[r, c] == (y if y > 0 else 0.0)
    assert np.array_equal(oracle.epilogue(ref), ref)  # no bias, no activation: identity


@pytest.mark.parametrize("act", [3, -1])
def test_rejects_unknown_activation(act):
    with pytest.raises(ValueError):
        oracle.epilogue(np.zeros((2, 2)), act=act)
