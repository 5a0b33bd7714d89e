"""Lloyd-Max scalar codebook for the Gaussian N(0, 1/d).

Method ([A] "Lloyd-Maxコードブックとは"; [C] "TurboQuantization: KV Cache
Compression", K-cache step 3): after the rotation each coordinate of a unit
vector is treated as N(0, 1/d); an 8-level (3-bit) minimum-MSE codebook for
that density is computed once, before inference, with no calibration data.
Lloyd-Max is an iteration, so this module runs it in the textbook order:

  1. decision thresholds are the midpoints of adjacent output levels;
  2. each output level is the conditional mean of the density on its cell;
  3. repeat until the levels stop moving.

Reading taken where the pages are silent:
  * The iteration runs on the standard normal N(0, 1) and is scaled by
    1/sqrt(d) at the end (the Gaussian family is closed under scaling, so
    this is the same fixed point as iterating on N(0, 1/d) directly).
  * Thresholds are the midpoints of the float64 levels, scaled, then rounded
    once to float32; levels are rounded once to float32 the same way.  The
    float32 values are the codebook both the encoder and the decoder use.
  * Level index = rank of the level in ascending order (0 = most negative).
"""

from __future__ import annotations

import math

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _upper_tail(x: float) -> float:
    """Q(x) = P(X > x) for X ~ N(0, 1), accurate in both tails."""
    if x == math.inf:
        return 0.0
    if x == -math.inf:
        return 1.0
    return 0.5 * math.erfc(x / _SQRT2)


def _cell_mass(a: float, b: float) -> float:
    """P(a < X <= b) computed from whichever tail keeps precision."""
    if a >= 0.0:
        return _upper_tail(a) - _upper_tail(b)
    if b <= 0.0:
        return _upper_tail(-b) - _upper_tail(-a)
    return 1.0 - _upper_tail(b) - _upper_tail(-a)


def _conditional_mean(a: float, b: float) -> float:
    """E[X | a < X <= b] = (phi(a) - phi(b)) / P(a < X <= b)."""
    return (_pdf(a) - _pdf(b)) / _cell_mass(a, b)


def lloyd_max_gaussian(levels: int = 8, tol: float = 1e-15, max_iter: int = 100000,
                       init: np.ndarray | None = None):
    """Run Lloyd-Max on N(0, 1).

    Returns ``(centroids, thresholds, iterations)`` in float64, ascending,
    ``len(thresholds) == levels - 1``.  ``init`` is any strictly increasing
    starting set (default: a symmetric uniform grid).
    """
    if levels < 2:
        raise ValueError("levels must be >= 2")
    if init is None:
        c = np.array([(k - (levels - 1) / 2.0) * (4.0 / levels) for k in range(levels)])
    else:
        c = np.array(init, dtype=np.float64)
        if c.shape != (levels,) or np.any(np.diff(c) <= 0):
            raise ValueError("init must be strictly increasing with `levels` entries")
    it = 0
    for it in range(1, max_iter + 1):
        t = [(c[k] + c[k + 1]) / 2.0 for k in range(levels - 1)]       # step 1
        edges = [-math.inf] + t + [math.inf]
        c_new = np.array([_conditional_mean(edges[k], edges[k + 1])    # step 2
                          for k in range(levels)])
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        if delta < tol:                                                # step 3
            break
    t = np.array([(c[k] + c[k + 1]) / 2.0 for k in range(levels - 1)])
    return c, t, it


def quantizer_mse(centroids: np.ndarray, thresholds: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0, 1), by integrating each cell exactly.

    For a cell (a, b] with level c:  E[(X-c)^2 1_cell] =
      [P + a*phi(a) - b*phi(b)] - 2c[phi(a) - phi(b)] + c^2 P,
    using E[X^2 1_cell] = P + a phi(a) - b phi(b).
    """
    edges = [-math.inf] + list(thresholds) + [math.inf]
    total = 0.0
    for k, c in enumerate(centroids):
        a, b = edges[k], edges[k + 1]
        p = _cell_mass(a, b)
        apa = 0.0 if math.isinf(a) else a * _pdf(a)
        bpb = 0.0 if math.isinf(b) else b * _pdf(b)
        ex2 = p + apa - bpb
        ex1 = _pdf(a) - _pdf(b)
        total += ex2 - 2.0 * c * ex1 + c * c * p
    return total


def codebook_fp32(head_dim: int = 128, bits: int = 3):
    """The codebook for N(0, 1/head_dim) as used by encoder and decoder.

    Returns ``(centroids_f32, thresholds_f32)``: ``2**bits`` levels and
    ``2**bits - 1`` thresholds, each rounded once from float64 to float32.
    """
    c, t, _ = lloyd_max_gaussian(1 << bits)
    s = math.sqrt(float(head_dim))
    return (np.array([x / s for x in c], dtype=np.float64).astype(np.float32),
            np.array([x / s for x in t], dtype=np.float64).astype(np.float32))
