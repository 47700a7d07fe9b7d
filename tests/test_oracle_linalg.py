"""Pins of the oracle's products and of the error metric."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.formats import (bf16_bits_to_f64, dequant_q4_k_f32, dequant_q4_k_f64,
                            dequant_q8_0_f32, f32_to_bf16_bits, pack_q4_k_block, row_bytes)
from oracle.linalg import (floored_rel_err, literal_rel_err_stats, matmul_bf16_x_f64,
                           matmul_f32_x_f64, matvec_exact, matvec_f64)
from synth import activations_f32, q4_k_weights, q8_0_weights
from tests.pins import check_integer_matvec, check_one_hot_columns


@pytest.mark.parametrize("fmt,cols", [("q8_0", 32), ("q8_0", 512), ("q4_k", 256), ("q4_k", 512)])
def test_fp64_matvec_within_rounding_bound_of_exact(fmt, cols):
    rng = np.random.default_rng(cols)
    rows = 4
    if fmt == "q8_0":
        w = dequant_q8_0_f32(q8_0_weights(rng, rows, cols), rows, cols)
    else:
        w = dequant_q4_k_f32(q4_k_weights(rng, rows, cols), rows, cols)
    x = activations_f32(rng, cols)
    y = matvec_f64(w, x)
    exact = matvec_exact(w, x)
    u = 2.0 ** -53
    for r in range(rows):
        bound = cols * u * float(np.sum(np.abs(w[r].astype(np.float64) * x))) * 1.01
        assert abs(Fraction(float(y[r])) - exact[r]) <= Fraction(bound)


def test_integer_matvec_special_case():
    assert check_integer_matvec(matvec_f64, dequant_q4_k_f64, pack_q4_k_block)


def test_one_hot_returns_columns():
    rng = np.random.default_rng(3)
    w = dequant_q4_k_f32(q4_k_weights(rng, 7, 512), 7, 512)
    assert check_one_hot_columns(matvec_f64, w)


def test_matmul_rows_equal_matvec_of_each_token():
    rng = np.random.default_rng(4)
    w = dequant_q4_k_f32(q4_k_weights(rng, 6, 256), 6, 256)
    xb = f32_to_bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    Y = matmul_bf16_x_f64(xb, w)
    for n in range(3):
        xn = bf16_bits_to_f64(xb[n]).astype(np.float32)   # bf16 is exact in fp32
        assert np.allclose(Y[n], matvec_f64(w, xn), rtol=0, atol=1e-12)
    # brute force on one entry
    exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(bf16_bits_to_f64(xb[1]), w[2]))
    assert abs(Fraction(float(Y[1, 2])) - exact) < Fraction(1, 10 ** 9)


def test_small_batch_matmul_brute_force_and_rows():
    """Every entry of the fp32-activation product against an exact Fraction
    dot product (within the fp64 rounding bound), on Q8_0 and Q4_K weights,
    and each token row against the matvec of that token."""
    rng = np.random.default_rng(6)
    for fmt, cols in (("q8_0", 64), ("q4_k", 256)):
        rows, n = 3, 4
        if fmt == "q8_0":
            w = dequant_q8_0_f32(q8_0_weights(rng, rows, cols), rows, cols)
        else:
            w = dequant_q4_k_f32(q4_k_weights(rng, rows, cols), rows, cols)
        X = np.stack([activations_f32(rng, cols) for _ in range(n)])
        Y = matmul_f32_x_f64(X, w)
        assert Y.shape == (n, rows)
        u = 2.0 ** -53
        for t in range(n):
            exact = matvec_exact(w, X[t])
            for r in range(rows):
                bound = cols * u * float(np.sum(np.abs(w[r].astype(np.float64) * X[t]))) * 1.01
                assert abs(Fraction(float(Y[t, r])) - exact[r]) <= Fraction(bound)
            assert np.allclose(Y[t], matvec_f64(w, X[t]), rtol=0, atol=1e-9)


def test_small_batch_matmul_integer_case_is_exact():
    """d = 1, dmin = 0, sc = 1: W holds the integers q, so with integer X every
    product is an exact integer sum (textbook integer matrix product)."""
    rng = np.random.default_rng(8)
    rows, cols, n = 5, 256, 3
    q = rng.integers(0, 16, size=(rows, cols))
    blob = b"".join(pack_q4_k_block(0x3C00, 0x0000, [1] * 8, [0] * 8, list(q[r])) for r in range(rows))
    w = dequant_q4_k_f32(np.frombuffer(blob, np.uint8), rows, cols)
    assert np.array_equal(w, q.astype(np.float32))
    X = rng.integers(-20, 21, size=(n, cols)).astype(np.float32)
    Y = matmul_f32_x_f64(X, w)
    assert np.array_equal(Y, (X.astype(np.int64) @ q.T).astype(np.float64))


def test_floored_metric_values():
    e, ok = floored_rel_err([3.1, 4.0], [3.0, 4.0])
    rho = np.sqrt((9 + 16) / 2)
    assert ok and abs(e - 0.1 / rho) < 1e-15
    # near-zero reference: floor applies
    e, ok = floored_rel_err([1e-3, 10.0], [0.0, 10.0])
    assert abs(e - 1e-3 / np.sqrt(50.0)) < 1e-15
    # large reference: plain relative error
    e, _ = floored_rel_err([0.0, 101.0], [0.0, 100.0])
    assert abs(e - 0.01) < 1e-15
    # non-finite output fails
    e, ok = floored_rel_err([np.nan, 1.0], [1.0, 1.0])
    assert not ok and e == float("inf")
    # per token row for matrices
    e, _ = floored_rel_err([[1.0, 1.0], [100.0, 101.0]], [[1.0, 1.0], [100.0, 100.0]])
    assert abs(e - 0.01) < 1e-15


def test_literal_stats():
    s = literal_rel_err_stats([1.0, 2.2, 0.0], [1.0, 2.0, 0.0], 0.05)
    assert abs(s["max"] - 0.1) < 1e-12 and s["above_tol"] == 1


def test_row_bytes_of_workload_shapes():
    assert row_bytes("q8_0", 512) == 544 and row_bytes("q8_0", 2048) == 2176
    assert row_bytes("q4_k", 2048) == 1152 and row_bytes("q4_k", 11008) == 6192
    with pytest.raises(ValueError):
        row_bytes("q4_k", 2047)
