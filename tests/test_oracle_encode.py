"""Pins of the oracle's key/value encoder."""
import math

import numpy as np
import pytest

from oracle import codebook_fp32, encode_k, encode_v, quantize_codes, fwht
from oracle.encode import residual_signs_from_codes, to_half_saturating
from oracle.codebook import lloyd_max_gaussian, quantizer_mse


def test_cell_search_is_nearest_centroid():
    c32, t32 = codebook_fp32(128, 3)
    rng = np.random.default_rng(0)
    y = rng.standard_normal(200_000) / math.sqrt(128) * 1.5
    idx = quantize_codes(y, t32)
    y32 = y.astype(np.float32).astype(np.float64)
    brute = np.argmin(np.abs(y32[:, None] - c32.astype(np.float64)[None, :]), axis=1)
    # away from ties the threshold search and brute-force nearest level agree
    dist = np.min(np.abs(y32[:, None] - t32.astype(np.float64)[None, :]), axis=1)
    far = dist > 1e-7
    np.testing.assert_array_equal(idx[far], brute[far])
    # ties go to the lower cell
    assert quantize_codes(np.array([float(t32[3])]), t32)[0] == 3
    assert quantize_codes(np.array([float(t32[0])]), t32)[0] == 0
    assert quantize_codes(np.array([float(t32[6]) * 1.01]), t32)[0] == 7


def test_norm_rotation_and_residual_identities():
    c32, t32 = codebook_fp32(128, 3)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 128)) * np.exp(rng.standard_normal(128))
    S = rng.standard_normal((128, 128)).astype(np.float32)
    enc = encode_k(x, c32, t32, S)
    np.testing.assert_allclose(enc["norm"], np.linalg.norm(x, axis=1), rtol=1e-14)
    # y is the rotated unit vector (fast transform, independent of the matrix)
    np.testing.assert_allclose(enc["y"], fwht(x / np.linalg.norm(x, axis=1)[:, None]), atol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(enc["y"], axis=1), 1.0, rtol=1e-13)
    # gamma measured in the rotated domain equals the original-domain residual
    yhat = c32.astype(np.float64)[enc["codes"].astype(int)]
    np.testing.assert_allclose(enc["gamma"], np.linalg.norm(enc["y"] - yhat, axis=1), rtol=1e-12)
    # z = S r, sign bit set for z >= 0
    np.testing.assert_allclose(enc["z"], enc["residual"] @ S.astype(np.float64).T, rtol=1e-12)
    np.testing.assert_array_equal(enc["signs"], (enc["z"] >= 0).astype(np.uint8))
    g2, z2, b2 = residual_signs_from_codes(x, enc["codes"], c32, S)
    np.testing.assert_allclose(g2, enc["gamma"], rtol=1e-13)
    np.testing.assert_array_equal(b2, enc["signs"])


def test_mean_squared_residual_matches_codebook_distortion():
    # For random directions the rotated coordinates are close to N(0, 1/d), so
    # E[gamma^2] is close to the standardised distortion of the codebook.
    c32, t32 = codebook_fp32(128, 3)
    c, t, _ = lloyd_max_gaussian(8)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((20000, 128))
    enc = encode_v(x, c32, t32)
    yhat = c32.astype(np.float64)[enc["codes"].astype(int)]
    g2 = np.sum((enc["y"] - yhat) ** 2, axis=1)
    assert abs(g2.mean() / quantizer_mse(c, t) - 1.0) < 0.03


def test_tiny_hand_worked_key():
    # d = m = 4, x = e0: u = e0, y = H e0 = (1/2, 1/2, 1/2, 1/2).  With the
    # N(0, 1/4) codebook the thresholds are (..., 0, 0.2503, 0.5250, ...), so
    # every y_i lies in cell 5 and yhat = c[5] (1, 1, 1, 1).  H^T yhat =
    # (2 c[5], 0, 0, 0), so r = (1 - 2 c[5], 0, 0, 0), gamma = 1 - 2 c[5].
    # With rows S = [e0; -e0; e1; 0]: z = (r0, -r0, 0, 0) -> bits 1, 0, 1, 1.
    c32, t32 = codebook_fp32(4, 3)
    S = np.array([[1, 0, 0, 0], [-1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 0, 0]], dtype=np.float32)
    enc = encode_k(np.array([[1.0, 0, 0, 0]]), c32, t32, S)
    np.testing.assert_array_equal(enc["codes"][0], [5, 5, 5, 5])
    r0 = 1.0 - 2.0 * float(c32[5])
    np.testing.assert_allclose(enc["residual"][0], [r0, 0, 0, 0], atol=1e-15)
    assert abs(enc["gamma"][0] - abs(r0)) < 1e-15
    np.testing.assert_array_equal(enc["signs"][0], [1, 0, 1, 1])
    assert enc["norm"][0] == 1.0


def test_zero_vector_and_scaling():
    c32, t32 = codebook_fp32(128, 3)
    S = np.random.default_rng(4).standard_normal((128, 128)).astype(np.float32)
    enc = encode_k(np.zeros((1, 128)), c32, t32, S)
    assert enc["norm"][0] == 0.0
    np.testing.assert_array_equal(enc["codes"][0], np.full(128, 3))
    # codes depend only on direction
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 128))
    a = encode_k(x, c32, t32, S)
    b = encode_k(x * 37.0, c32, t32, S)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["signs"], b["signs"])


def test_half_storage_rounds_to_nearest_even_and_saturates():
    assert to_half_saturating(1.0 + 2.0 ** -11)[()] == np.float16(1.0)          # tie -> even
    assert to_half_saturating(1.0 + 3 * 2.0 ** -11)[()] == np.float16(1.0 + 2.0 ** -9)
    assert to_half_saturating(1e6)[()] == np.float16(65504.0)
    v = np.random.default_rng(6).uniform(1, 1000, 1000)
    np.testing.assert_array_equal(to_half_saturating(v), v.astype(np.float16))
