"""Pins of the oracle's QJL generator and of the estimator it serves."""
import math

import pytest

import numpy as np
from scipy import stats

from golden_util import read_rows
from oracle import codebook_fp32, dequant_k, encode_k
from oracle.qjl import gaussian_matrix, qjl_alpha, splitmix64_stream


def test_splitmix64_published_vectors():
    rows = read_rows("splitmix64_vectors.txt")
    by_seed = {}
    for seed, idx, val in rows:
        by_seed.setdefault(int(seed), {})[int(idx)] = int(val)
    for seed, vals in by_seed.items():
        out = splitmix64_stream(seed, max(vals) + 1)
        for i, v in vals.items():
            assert out[i] == v


def test_gaussian_matrix_is_standard_normal():
    S = gaussian_matrix(42, 128, 128).astype(np.float64).ravel()
    n = S.size
    assert abs(S.mean()) < 4 / math.sqrt(n)
    assert abs(S.var() - 1.0) < 4 * math.sqrt(2.0 / n)
    assert stats.kstest(S, "norm").pvalue > 1e-3
    assert gaussian_matrix(42).dtype == np.float32
    np.testing.assert_array_equal(gaussian_matrix(42), gaussian_matrix(42))
    assert not np.array_equal(gaussian_matrix(42), gaussian_matrix(43))
    # rows are uncorrelated
    M = gaussian_matrix(7).astype(np.float64)
    C = np.corrcoef(M)
    off = C[~np.eye(128, dtype=bool)]
    assert np.abs(off).max() < 6 / math.sqrt(128)


def _estimate_stats(draws=3000, seed=11):
    """Over independent S: <q, k~> with k~ from encode_k + dequant_k (stored
    half scalars), against the exact <q, x>."""
    d = m = 128
    rng = np.random.default_rng(seed)
    c32, t32 = codebook_fp32(d, 3)
    x = rng.standard_normal(d) * 3.0
    x[[5, 77]] *= 20
    q = rng.standard_normal(d)
    est = np.empty(draws)
    for i in range(draws):
        S = rng.standard_normal((m, d)).astype(np.float32)
        enc = encode_k(x[None], c32, t32, S)
        kt = dequant_k(enc["codes"], enc["signs"], enc["norm_f16"], enc["gamma_f16"], c32, S)
        est[i] = kt[0] @ q
    r = enc["residual"][0]
    n = float(enc["norm_f16"][0])
    return est, float(x @ q), n, r, q


def test_qjl_estimator_variance_at_128_rows():
    # one 128-row S per draw, 3,000 draws: the per-draw variance at m = 128
    est, exact, n, r, q = _estimate_stats()
    se = est.std(ddof=1) / math.sqrt(est.size)
    # the half-precision norm moves the mean by at most 2^-11 relative
    assert abs(est.mean() - exact) < 4 * se + abs(exact) * 2.0 ** -11, (est.mean(), exact, se)
    m = 128
    var_theory = n * n * ((math.pi / 2) * (q @ q) * (r @ r) - (q @ r) ** 2) / m
    rel = est.var(ddof=1) / var_theory
    # the sample variance of 3000 draws is within ~ +-10 % (4 sd of its ratio)
    assert 0.85 < rel < 1.15, rel


def test_alpha_value():
    assert qjl_alpha(128) == math.sqrt(math.pi / 2) / 128


@pytest.mark.parametrize("pair", [0, 1, 2])
def test_qjl_estimator_unbiased_over_20000_draws(pair):
    """Unbiasedness over 20,000 independent 128 x 128 draws of S for three
    (x, q) pairs.  The draws are stacked: encode_k and dequant_k are called
    with the rows of 100 draws at once (m = 12,800).  The estimator is linear
    in the rows, and qjl_alpha(m) = sqrt(pi/2)/m, so each call returns the mean
    of its 100 per-draw estimates.  The 200 batch means must average to <q, x>
    within 4 standard errors, and their variance must match the closed form
    n^2 ((pi/2)|q|^2|r|^2 - <q, r>^2) / m at m = 12,800."""
    d = 128
    per_batch, batches = 100, 200
    rng = np.random.default_rng(100 + pair)
    c32, t32 = codebook_fp32(d, 3)
    x = rng.standard_normal(d) * (1.0 + 4.0 * pair)
    x[rng.choice(d, 2 + pair, replace=False)] *= 20.0
    q = rng.standard_normal(d)
    if pair == 2:  # a query nearly aligned with the key
        q = 0.2 * q + x / np.linalg.norm(x) * 8.0
    est = np.empty(batches)
    for i in range(batches):
        S = rng.standard_normal((d * per_batch, d), dtype=np.float32)
        enc = encode_k(x[None], c32, t32, S)
        kt = dequant_k(enc["codes"], enc["signs"], enc["norm_f16"], enc["gamma_f16"], c32, S)
        est[i] = kt[0] @ q
    exact = float(x @ q)
    n = float(enc["norm_f16"][0])
    r = enc["residual"][0]
    se = est.std(ddof=1) / math.sqrt(batches)
    # the half-precision norm moves the mean by at most 2^-11 relative
    assert abs(est.mean() - exact) < 4 * se + abs(exact) * 2.0 ** -11, (est.mean(), exact, se)
    m = d * per_batch
    var_theory = n * n * ((math.pi / 2) * (q @ q) * (r @ r) - (q @ r) ** 2) / m
    rel = est.var(ddof=1) / var_theory
    # sample variance of 200 batch means: within 4 sd (sqrt(2/199) = 10 %)
    assert 0.6 < rel < 1.4, rel
