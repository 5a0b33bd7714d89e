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


# ---- the exact marginal of one coordinate of a random unit vector -----------
# The pages ([A] "Lloyd-Maxコードブックとは") fit the codebook to N(0, 1/d), the
# large-d limit of one coordinate of a uniformly random unit vector in R^d.
# The exact marginal has density f(y) = C_d (1 - y^2)^((d-3)/2) on (-1, 1),
# C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)), and Y^2 ~ Beta(1/2, (d-1)/2).
# The variant below runs the same Lloyd-Max iteration on that density (cell
# masses and moments from the regularised incomplete beta function and the
# antiderivative of y (1 - y^2)^k); it is a reference, not the codebook the
# method uses.

def sphere_marginal_pdf(y: float, d: int) -> float:
    if abs(y) >= 1.0:
        return 0.0
    logc = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
    return math.exp(logc + 0.5 * (d - 3) * math.log1p(-y * y))


def _sphere_cdf(y: float, d: int) -> float:
    """P(Y <= y): 1/2 + sign(y) I_{y^2}(1/2, (d-1)/2) / 2."""
    import scipy.special
    if y <= -1.0:
        return 0.0
    if y >= 1.0:
        return 1.0
    half = 0.5 * float(scipy.special.betainc(0.5, (d - 1) / 2.0, y * y))
    return 0.5 + half if y >= 0.0 else 0.5 - half


def _sphere_first_moment(a: float, b: float, d: int) -> float:
    """Integral of y f(y) over (a, b]: C_d [(1-a^2)^(k+1) - (1-b^2)^(k+1)] / (2 (k+1)), k = (d-3)/2."""
    k1 = 0.5 * (d - 1)
    logc = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
    ua = 0.0 if abs(a) >= 1.0 else math.exp(k1 * math.log1p(-a * a))
    ub = 0.0 if abs(b) >= 1.0 else math.exp(k1 * math.log1p(-b * b))
    return math.exp(logc) * (ua - ub) / (2.0 * k1)


def _sphere_second_moment(a: float, b: float, d: int) -> float:
    """Integral of y^2 f(y) over (a, b]: with X = Y^2 ~ Beta(1/2, (d-1)/2),
    E[X 1{X <= s}] = I_s(3/2, (d-1)/2) / d, split at 0 by symmetry."""
    import scipy.special

    def upto(y):  # integral of y^2 f over [0, y] for y >= 0
        y = min(y, 1.0)
        return 0.5 * float(scipy.special.betainc(1.5, (d - 1) / 2.0, y * y)) / d

    def signed(y):  # integral over (-1, y]
        return 1.0 / (2 * d) + (upto(y) if y >= 0.0 else -upto(-y))

    a, b = max(a, -1.0), min(b, 1.0)
    return signed(b) - signed(a)


def lloyd_max_sphere(levels: int, d: int, tol: float = 1e-15, max_iter: int = 100000):
    """Lloyd-Max on the exact marginal f above, in the same order as
    ``lloyd_max_gaussian`` (midpoint thresholds, conditional-mean levels,
    repeat).  Returns ``(centroids, thresholds, iterations)`` in float64 on
    the unit-vector scale (no further 1/sqrt(d) scaling)."""
    if levels < 2 or d < 3:
        raise ValueError("levels >= 2 and d >= 3")
    s = 1.0 / math.sqrt(d)
    c = np.array([(k - (levels - 1) / 2.0) * (4.0 / levels) * s for k in range(levels)])
    c = np.clip(c, -0.99, 0.99)
    it = 0
    for it in range(1, max_iter + 1):
        t = [(c[k] + c[k + 1]) / 2.0 for k in range(levels - 1)]
        edges = [-1.0] + t + [1.0]
        c_new = np.array([_sphere_first_moment(edges[k], edges[k + 1], d) /
                          (_sphere_cdf(edges[k + 1], d) - _sphere_cdf(edges[k], d)) for k in range(levels)])
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        if delta < tol:
            break
    t = np.array([(c[k] + c[k + 1]) / 2.0 for k in range(levels - 1)])
    return c, t, it


def quantizer_mse_sphere(centroids: np.ndarray, thresholds: np.ndarray, d: int) -> float:
    """E[(Y - Q(Y))^2] under the exact marginal, cell by cell:
    E[Y^2 1_cell] - 2 c E[Y 1_cell] + c^2 P(cell)."""
    edges = [-1.0] + list(thresholds) + [1.0]
    total = 0.0
    for k, c in enumerate(centroids):
        a, b = edges[k], edges[k + 1]
        p = _sphere_cdf(b, d) - _sphere_cdf(a, d)
        total += _sphere_second_moment(a, b, d) - 2.0 * c * _sphere_first_moment(a, b, d) + c * c * p
    return total
