"""Pins of the oracle's Lloyd-Max codebook against mathematics and Max (1960)."""
import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle.codebook import codebook_fp32, lloyd_max_gaussian, quantizer_mse
from golden_util import read_rows


def _quad_cell_mean(a, b):
    num = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    den = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-15, epsrel=1e-13)[0]
    return num / den


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_fixed_point_conditions(levels):
    c, t, _ = lloyd_max_gaussian(levels)
    # thresholds are exact midpoints of adjacent levels
    np.testing.assert_array_equal(t, (c[:-1] + c[1:]) / 2.0)
    # levels are conditional means of N(0,1) on their cells (numerical quadrature)
    edges = [-np.inf] + list(t) + [np.inf]
    for k in range(levels):
        assert abs(c[k] - _quad_cell_mean(edges[k], edges[k + 1])) < 1e-9


@pytest.mark.parametrize("levels", [2, 4, 8])
def test_symmetric_and_ascending(levels):
    c, t, _ = lloyd_max_gaussian(levels)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(c, -c[::-1], atol=1e-15)
    np.testing.assert_allclose(t, -t[::-1], atol=1e-15)


def test_two_levels_closed_form():
    # Two-level Gaussian quantizer: levels +-E|X| = +-sqrt(2/pi), threshold 0,
    # MSE 1 - 2/pi.
    c, t, _ = lloyd_max_gaussian(2)
    np.testing.assert_allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=1e-14)
    assert t[0] == 0.0
    assert abs(quantizer_mse(c, t) - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("name,levels", [("max1960_gaussian_8level.txt", 8),
                                         ("max1960_gaussian_4level.txt", 4)])
def test_matches_max_1960_table(name, levels):
    c, t, _ = lloyd_max_gaussian(levels)
    pos_c = c[levels // 2:]
    pos_t = t[levels // 2:]
    for kind, idx, val in read_rows(name):
        idx = int(idx)
        digits = len(val.split(".")[1])
        # the 1960 table is rounded by hand and is off by up to one unit in
        # its last printed digit (e.g. 0.5006 for 0.500550)
        half_unit = 1.0 * 10 ** (-digits) + 1e-12
        if kind == "level":
            assert abs(pos_c[idx - 1] - float(val)) <= half_unit, (kind, idx, pos_c[idx - 1], val)
        elif kind == "threshold":
            assert abs(pos_t[idx - 1] - float(val)) <= half_unit, (kind, idx, pos_t[idx - 1], val)
        else:
            assert abs(quantizer_mse(c, t) - float(val)) <= half_unit


def test_mse_closed_form_matches_quadrature_and_monte_carlo():
    c, t, _ = lloyd_max_gaussian(8)
    mse = quantizer_mse(c, t)
    edges = [-np.inf] + list(t) + [np.inf]
    q = sum(integrate.quad(lambda x, ck=ck: (x - ck) ** 2 * stats.norm.pdf(x), a, b,
                           epsabs=1e-14)[0]
            for ck, a, b in zip(c, edges[:-1], edges[1:]))
    assert abs(mse - q) < 1e-10
    rng = np.random.default_rng(7)
    x = rng.standard_normal(2_000_000)
    nearest = c[np.argmin(np.abs(x[:, None] - c[None, :]), axis=1)]
    err = (x - nearest) ** 2
    assert abs(err.mean() - mse) < 4 * err.std() / math.sqrt(x.size)


def test_unique_fixed_point_from_any_start():
    ref, _, _ = lloyd_max_gaussian(8)
    rng = np.random.default_rng(3)
    for _ in range(5):
        init = np.sort(rng.uniform(-5, 5, 8))
        c, _, _ = lloyd_max_gaussian(8, init=init)
        np.testing.assert_allclose(c, ref, atol=1e-12)


def test_fp32_codebook_is_scaled_and_rounded_once():
    c, t, _ = lloyd_max_gaussian(8)
    c32, t32 = codebook_fp32(128, 3)
    assert c32.dtype == np.float32 and t32.dtype == np.float32
    np.testing.assert_array_equal(c32, np.array([x / math.sqrt(128) for x in c]).astype(np.float32))
    np.testing.assert_array_equal(t32, np.array([x / math.sqrt(128) for x in t]).astype(np.float32))
    # N(0, 1/d) scaling: back in standard units the fp32 levels are within one
    # fp32 rounding of the float64 fixed point
    np.testing.assert_allclose(c32.astype(np.float64) * math.sqrt(128), c, rtol=6e-8)


# ---- the exact sphere-marginal variant ---------------------------------------
from oracle.codebook import (lloyd_max_sphere, quantizer_mse_sphere, sphere_marginal_pdf, _sphere_cdf,
                             _sphere_first_moment, _sphere_second_moment)


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_sphere_codebook_in_three_dimensions_is_the_uniform_quantizer(levels):
    """For d = 3 a coordinate of a random unit vector is uniform on [-1, 1]
    (Archimedes), whose minimum-MSE quantizer is the uniform one: levels
    -1 + (2k+1)/L, thresholds -1 + 2k/L, MSE = 1/(3 L^2)."""
    c, t, _ = lloyd_max_sphere(levels, 3)
    k = np.arange(levels)
    np.testing.assert_allclose(c, -1 + (2 * k + 1) / levels, atol=1e-12)
    np.testing.assert_allclose(t, -1 + 2 * (k[:-1] + 1) / levels, atol=1e-12)
    assert abs(quantizer_mse_sphere(c, t, 3) - 1 / (3 * levels ** 2)) < 1e-14


def test_sphere_moments_match_quadrature():
    """Cell masses and first / second moments from the closed forms against
    adaptive quadrature of the density."""
    import scipy.integrate
    rng = np.random.default_rng(0)
    for d in (3, 5, 16, 128):
        total = scipy.integrate.quad(lambda y: sphere_marginal_pdf(y, d), -1, 1)[0]
        assert abs(total - 1.0) < 1e-10
        for _ in range(5):
            a, b = np.sort(rng.uniform(-1, 1, 2) * (1.0 if d < 16 else 0.4))
            m0 = scipy.integrate.quad(lambda y: sphere_marginal_pdf(y, d), a, b, epsabs=1e-14)[0]
            m1 = scipy.integrate.quad(lambda y: y * sphere_marginal_pdf(y, d), a, b, epsabs=1e-14)[0]
            m2 = scipy.integrate.quad(lambda y: y * y * sphere_marginal_pdf(y, d), a, b, epsabs=1e-14)[0]
            assert abs(_sphere_cdf(b, d) - _sphere_cdf(a, d) - m0) < 1e-11
            assert abs(_sphere_first_moment(a, b, d) - m1) < 1e-11
            assert abs(_sphere_second_moment(a, b, d) - m2) < 1e-11


@pytest.mark.parametrize("levels", [4, 8, 16])
def test_sphere_codebook_is_a_lloyd_max_fixed_point(levels):
    """At d = 128: every threshold is the midpoint of its levels and every
    level the conditional mean of its cell (recomputed by quadrature)."""
    import scipy.integrate
    d = 128
    c, t, _ = lloyd_max_sphere(levels, d)
    np.testing.assert_allclose(t, (c[:-1] + c[1:]) / 2, rtol=0, atol=1e-15)
    edges = [-1.0] + list(t) + [1.0]
    for k in range(levels):
        a, b = edges[k], edges[k + 1]
        m0 = scipy.integrate.quad(lambda y: sphere_marginal_pdf(y, d), a, b, epsabs=1e-15)[0]
        m1 = scipy.integrate.quad(lambda y: y * sphere_marginal_pdf(y, d), a, b, epsabs=1e-15)[0]
        assert abs(m1 / m0 - c[k]) < 1e-10


def test_sphere_codebook_tends_to_the_gaussian_one_and_beats_it():
    """sqrt(d) times the sphere levels approach the N(0, 1) Lloyd-Max levels
    as d grows (the coordinate tends to N(0, 1/d)); at every d the sphere
    codebook has the lower exact MSE under the true marginal (its density
    is log-concave, so the fixed point is the optimum)."""
    g, tg, _ = lloyd_max_gaussian(8)
    prev = None
    for d in (16, 128, 1024, 8192):
        c, t, _ = lloyd_max_sphere(8, d)
        err = np.max(np.abs(c * np.sqrt(d) - g) / np.abs(g))
        if prev is not None:
            assert err < prev
        prev = err
        assert quantizer_mse_sphere(c, t, d) <= quantizer_mse_sphere(g / np.sqrt(d), tg / np.sqrt(d), d)
    assert prev < 5e-4


def test_sphere_codebook_mse_by_monte_carlo():
    """20,000 random unit vectors in R^128: the empirical per-coordinate MSE
    of the sphere codebook matches its exact MSE within 4 standard errors."""
    d = 128
    c, t, _ = lloyd_max_sphere(8, d)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20000, d))
    y = (x / np.linalg.norm(x, axis=1, keepdims=True)).ravel()
    err2 = (y - c[np.searchsorted(t, y)]) ** 2
    se = err2.std() / np.sqrt(err2.size)
    assert abs(err2.mean() - quantizer_mse_sphere(c, t, d)) < 4 * se
