"""8-level Lloyd-Max quantizer of the standard normal (test infrastructure only).

[SV] "14 попыток, которые провалились" describes the turbo3 dequant as a lookup
into a small LUT of quantizer levels held in constant memory; the LUT3 cache
format fills its 8-entry LUT with the minimum-MSE (Lloyd-Max) levels of N(0,1).

Lloyd's fixed-point iteration for a density f: decision thresholds sit halfway
between adjacent levels, and each level is the conditional mean of its cell,
    t_k = (y_k + y_{k+1}) / 2,
    y_k = E[X | t_{k-1} < X <= t_k] = (phi(t_{k-1}) - phi(t_k)) / (Phi(t_k) - Phi(t_{k-1}))
for the standard normal (phi = density, Phi = distribution function). The
quantizer is symmetric, so only the four positive levels are iterated, with the
innermost threshold fixed at 0 and the outermost at +infinity.
"""
from __future__ import annotations

import math

import numpy as np


def _phi(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x: float) -> float:
    if math.isinf(x):
        return 1.0 if x > 0 else 0.0
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def levels(n_pos: int = 4, iters: int = 2000, tol: float = 1e-15):
    """Positive levels and thresholds of the 2*n_pos-level Lloyd-Max quantizer of N(0,1).

    Returns (levels, thresholds, mse): ``levels`` y_1 < ... < y_n (float64),
    ``thresholds`` t_1 < ... < t_{n-1} between them, and the mean squared error
    of the full symmetric quantizer.
    """
    # start from equally spaced levels
    y = np.array([0.5 + k for k in range(n_pos)], dtype=np.float64)
    for _ in range(iters):
        t = [0.0] + [(y[k] + y[k + 1]) / 2.0 for k in range(n_pos - 1)] + [math.inf]
        new = np.array([(_phi(t[k]) - _phi(t[k + 1])) / (_Phi(t[k + 1]) - _Phi(t[k]))
                        for k in range(n_pos)])
        done = np.max(np.abs(new - y)) < tol
        y = new
        if done:
            break
    t = [0.0] + [(y[k] + y[k + 1]) / 2.0 for k in range(n_pos - 1)] + [math.inf]
    # MSE = E[X^2] - sum_k P_k y_k^2 for a centroid quantizer (both halves)
    mse = 1.0 - 2.0 * sum((_Phi(t[k + 1]) - _Phi(t[k])) * y[k] ** 2 for k in range(n_pos))
    return y, np.array(t[1:-1]), mse


def lut3_magnitudes_f16() -> np.ndarray:
    """The four LUT magnitudes as float16 (round to nearest even from float64)."""
    y, _, _ = levels(4)
    return y.astype(np.float16)
