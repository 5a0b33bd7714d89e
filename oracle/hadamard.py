"""Walsh-Hadamard rotation.

Method ([A] "Walsh-Hadamard Transform（WHT）の役割"; [C] "TurboQuantization",
K-cache step 2): the rotation spreads outlier channels over all coordinates;
it is orthogonal and built from additions and subtractions only, with an
FFT-like divide-and-conquer structure.

Readings taken where the pages are silent:
  * Orthonormal scaling H = H_d / sqrt(d) (the pages call it orthogonal), so
    H is symmetric and its own inverse: H = H^T = H^{-1}.
  * Sylvester (natural) ordering, H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]],
    with no random sign diagonal (the pages list none).
"""

from __future__ import annotations

import math

import numpy as np


def sylvester_hadamard(d: int) -> np.ndarray:
    """Explicit orthonormal Sylvester matrix H_d / sqrt(d), float64, by its
    recursive definition."""
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(d)


def fwht(x: np.ndarray) -> np.ndarray:
    """Fast transform along the last axis: log2(d) butterfly stages of
    (a, b) -> (a + b, a - b), then one 1/sqrt(d) scale.  Same result as
    ``x @ sylvester_hadamard(d)`` (H is symmetric)."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError("last dimension must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y / math.sqrt(d)
