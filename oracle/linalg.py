"""Reference products and the error metric (oracle; test infrastructure only)."""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .formats import bf16_bits_to_f64


def matvec_f64(w32: np.ndarray, x32: np.ndarray) -> np.ndarray:
    """y[r] = sum_k w[r, k] x[k] in fp64 from the fp32 dequantized weights and
    the fp32 activations (culpeo.ws naive-implementation post: matvec takes
    w [r, c] and x [c] and returns [r]; "GGUF Inferencer in R", section 5.2:
    the projections are the input times the transposed weight matrix)."""
    return np.asarray(w32, dtype=np.float64) @ np.asarray(x32, dtype=np.float64)


def matmul_bf16_x_f64(x_bf16_bits: np.ndarray, w32: np.ndarray) -> np.ndarray:
    """Y[n, r] = sum_k X[n, k] W[r, k] in fp64, X given as bf16 bit patterns
    [n_tokens, K] and W as the fp32 dequant [rows, K]. Prefill is the decode
    math applied to the whole prompt as one matrix ("GGUF Inferencer in R",
    section 1 and section 4). W is NOT rounded to bf16 here: that rounding is
    the approximation the bf16 tolerance covers."""
    X = bf16_bits_to_f64(x_bf16_bits)
    return X @ np.asarray(w32, dtype=np.float64).T


def matmul_f32_x_f64(x32: np.ndarray, w32: np.ndarray) -> np.ndarray:
    """Y[n, r] = sum_k X[n, k] W[r, k] in fp64, X fp32 [n_tokens, K] and W the
    fp32 dequant [rows, K]: the decode matvec applied to several activation
    vectors at once (culpeo.ws naive-implementation post, matvec of w [r, c]
    by x [c]; "GGUF Inferencer in R", section 1: prefill runs the same math
    on a matrix of tokens). Row n of Y is the matvec of token n."""
    X = np.asarray(x32, dtype=np.float32).astype(np.float64)
    return X @ np.asarray(w32, dtype=np.float64).T


def matvec_exact(w, x) -> list:
    """Exact y = W x with Fractions, for tiny shapes (brute force)."""
    w = np.asarray(w)
    x = np.asarray(x)
    rows, cols = w.shape
    xf = [Fraction(float(v)) for v in x]
    out = []
    for r in range(rows):
        acc = Fraction(0)
        for k in range(cols):
            acc += Fraction(float(w[r, k])) * xf[k]
        out.append(acc)
    return out


def floored_rel_err(y, y_ref):
    """Per-output relative error with a floor, per output vector.

    For one output vector (a GEMV result, or one token row of a prefill
    result): rho = rms(y_ref); e_i = |y_i - y_ref_i| / max(|y_ref_i|, rho).
    Returns (max e over everything, all y finite). A bare |dy|/|y_ref| is
    ill-posed for outputs that cancel to near zero, which any correct fp32 or
    bf16 summation order hits on a few outputs; the floor at the vector's rms
    keeps the bound meaningful there.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {y_ref.shape}")
    if y.size == 0:
        return 0.0, True
    y2 = y.reshape(-1, y.shape[-1]) if y.ndim > 1 else y.reshape(1, -1)
    r2 = y_ref.reshape(y2.shape)
    rho = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    denom = np.maximum(np.abs(r2), rho)
    denom = np.where(denom == 0, 1.0, denom)
    e = np.abs(y2 - r2) / denom
    finite = bool(np.all(np.isfinite(y2)))
    return float(np.max(e)) if finite else float("inf"), finite


def literal_rel_err_stats(y, y_ref, tol: float):
    """The un-floored |dy| / |y_ref|: max, 99.9th percentile, count above tol
    (reported beside the floored metric, not used as the gate)."""
    y = np.asarray(y, dtype=np.float64).ravel()
    y_ref = np.asarray(y_ref, dtype=np.float64).ravel()
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.abs(y - y_ref) / np.abs(y_ref)
    e = np.where(np.isnan(e), 0.0, e)
    return {"max": float(np.max(e)) if e.size else 0.0,
            "p99_9": float(np.percentile(e, 99.9)) if e.size else 0.0,
            "above_tol": int(np.sum(e > tol))}
