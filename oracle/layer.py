"""The steps either side of the decode GEMVs (oracle; test infrastructure only).

"GGUF Inferencer in R", section 5.2: the layer normalizes its input with
RMSN(v) = norm * v / sqrt(mean(v^2) + epsilon) before the q/k/v and before
the gate/up projections (5.2.1, 5.2.2), activates with SiLU(G) * U where
SiLU(x) = x / (1 + exp(-x)) (5.2.2), and adds each projection's output back
to its input (the residual adds after the output and down projections). All
in fp64 from the fp32 inputs.
"""

from __future__ import annotations

import numpy as np


def rmsnorm_f64(v, norm_w, eps: float) -> np.ndarray:
    """RMSN(v) = norm_w * v / sqrt(mean(v^2) + eps)."""
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(norm_w, dtype=np.float64)
    return w * v / np.sqrt(np.mean(v * v) + float(eps))


def silu_f64(x) -> np.ndarray:
    """SiLU(x) = x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_f64(g, u) -> np.ndarray:
    """The gated activation SiLU(G) * U."""
    return silu_f64(g) * np.asarray(u, dtype=np.float64)
