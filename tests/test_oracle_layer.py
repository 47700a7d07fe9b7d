"""Pins of the oracle's RMSN and SiLU against closed forms."""

import math

import numpy as np

from oracle.layer import rmsnorm_f64, silu_f64, swiglu_f64


def test_rmsnorm_hand_example():
    # v = (3, 4): mean of squares 12.5
    got = rmsnorm_f64([3.0, 4.0], [1.0, 2.0], 0.0)
    r = math.sqrt(12.5)
    assert np.allclose(got, [3 / r, 8 / r], rtol=0, atol=1e-15)


def test_rmsnorm_constant_vector_and_epsilon():
    for c in (0.5, -3.0, 1e3):
        v = np.full(64, c)
        assert np.allclose(rmsnorm_f64(v, np.ones(64), 0.0), np.sign(c), rtol=0, atol=1e-15)
        assert np.allclose(rmsnorm_f64(v, np.ones(64), 0.25), c / math.sqrt(c * c + 0.25), rtol=1e-15)
    # the epsilon keeps a zero vector finite
    assert np.array_equal(rmsnorm_f64(np.zeros(8), np.ones(8), 1e-6), np.zeros(8))


def test_rmsnorm_is_scale_invariant_without_epsilon():
    rng = np.random.default_rng(3)
    v, w = rng.standard_normal(300), rng.standard_normal(300)
    assert np.allclose(rmsnorm_f64(v, w, 0.0), rmsnorm_f64(7.5 * v, w, 0.0), rtol=1e-13)
    # and its output has rms 1 when the weights are 1
    out = rmsnorm_f64(v, np.ones(300), 0.0)
    assert abs(math.sqrt(np.mean(out * out)) - 1.0) < 1e-14


def test_silu_closed_forms():
    assert silu_f64(0.0) == 0.0
    # sigmoid(ln 3) = 3/4
    assert abs(silu_f64(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    x = np.linspace(-20, 20, 81)
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    assert np.allclose(silu_f64(x) - silu_f64(-x), x, rtol=0, atol=1e-13)
    # large arguments: silu(x) -> x for x >> 0, -> 0 for x << 0
    assert abs(silu_f64(60.0) - 60.0) < 1e-20 * 1e10
    assert abs(silu_f64(-60.0)) < 1e-24


def test_swiglu_is_silu_times_up():
    g = np.array([-2.0, 0.0, 1.0, 3.0])
    u = np.array([5.0, 7.0, -1.0, 0.5])
    assert np.allclose(swiglu_f64(g, u), g / (1 + np.exp(-g)) * u, rtol=0, atol=1e-15)
