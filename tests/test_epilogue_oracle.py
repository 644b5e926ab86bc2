"""Pins of the epilogue oracle (oracle/epilogue.py) against facts of the
activations' mathematics: textbook values, odd-symmetry identities that each
form satisfies exactly, limits, and the Lipschitz constants used by the GPU
tolerance (Bolt page, epilogue fusion)."""
import math

import numpy as np
import pytest

from oracle import epilogue as ep


def test_textbook_values():
    # Phi(1) = 0.8413447460685429 (standard normal table), so gelu(1) = Phi(1)
    assert ep.activation("gelu", np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    # Phi(-1) = 0.15865525393145707: gelu(-1) = -Phi(-1)
    assert ep.activation("gelu", np.array([-1.0]))[0] == pytest.approx(-0.15865525393145707, rel=1e-14)
    # sigmoid(1) = e / (1 + e) = 0.7310585786300049
    assert ep.activation("silu", np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    # the tanh form at 1: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715)) = 0.8411919906082768
    assert ep.activation("gelu_tanh", np.array([1.0]))[0] == pytest.approx(0.8411919906082768, rel=1e-14)
    assert list(ep.activation("relu", np.array([-2.5, 0.0, 3.25]))) == [0.0, 0.0, 3.25]
    for a in ("gelu", "gelu_tanh", "silu", "relu", "none"):
        assert ep.activation(a, np.array([0.0]))[0] == 0.0


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu", "relu"])
def test_odd_part_is_identity(act):
    """x * F(x) with F(x) + F(-x) = 1 (Phi, the tanh form, sigmoid, the
    step function) gives act(x) - act(-x) = x."""
    x = np.linspace(-9, 9, 2001)
    d = ep.activation(act, x) - ep.activation(act, -x)
    assert np.allclose(d, x, rtol=0, atol=4e-15 * np.maximum(1.0, np.abs(x)))


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu"])
def test_limits(act):
    big = np.array([30.0, 60.0])
    assert np.allclose(ep.activation(act, big), big, rtol=1e-12)
    assert np.all(np.abs(ep.activation(act, -big)) < 1e-10)


def test_gelu_tanh_is_close_to_gelu():
    # the tanh form approximates x Phi(x) to about 1e-3 absolute on [-6, 6]
    x = np.linspace(-6, 6, 4001)
    assert np.max(np.abs(ep.activation("gelu", x) - ep.activation("gelu_tanh", x))) < 1e-3


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu", "relu"])
def test_lipschitz_constants_bound_the_slope(act):
    x = np.linspace(-12, 12, 200001)
    y = ep.activation(act, x)
    slope = np.abs(np.diff(y) / np.diff(x))
    assert slope.max() <= ep.LIPSCHITZ[act]
    assert slope.max() > ep.LIPSCHITZ[act] - 0.01   # and is not loose


def test_epilogue_terms():
    rng = np.random.default_rng(3)
    acc = rng.normal(size=(5, 7))
    c = rng.normal(size=(5, 7))
    bias = rng.normal(size=7)
    # identity epilogue returns the product unchanged
    assert np.array_equal(ep.epilogue(acc), acc)
    # dyadic alpha, beta: every term exact, compare with the sum written out per element
    out = ep.epilogue(acc, 2.0, 0.5, c, bias, "relu")
    for i in range(5):
        for j in range(7):
            v = 2.0 * acc[i, j] + 0.5 * c[i, j] + bias[j]
            assert out[i, j] == (v if v > 0 else 0.0)
    # beta == 0 never reads C (NaN there stays out of the result)
    assert np.isfinite(ep.epilogue(acc, 1.0, 0.0, np.full_like(acc, np.nan), bias, "gelu")).all()
