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
