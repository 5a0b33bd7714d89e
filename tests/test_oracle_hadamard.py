"""Pins of the oracle's Walsh-Hadamard rotation."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle.hadamard import fwht, sylvester_hadamard


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_matches_library_and_is_orthonormal_involution(d):
    h = sylvester_hadamard(d)
    np.testing.assert_array_equal(h * math.sqrt(d), scipy.linalg.hadamard(d))
    np.testing.assert_allclose(h @ h, np.eye(d), atol=1e-12)
    np.testing.assert_array_equal(h, h.T)


@pytest.mark.parametrize("d", [2, 4, 8, 16])
def test_entries_by_bit_parity(d):
    # Sylvester order: H[i, j] = (-1)^popcount(i & j) / sqrt(d)
    h = sylvester_hadamard(d)
    for i in range(d):
        for j in range(d):
            assert h[i, j] == (-1) ** bin(i & j).count("1") / math.sqrt(d)


@pytest.mark.parametrize("d", [1, 2, 8, 128])
def test_fast_transform_equals_matrix(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    np.testing.assert_allclose(fwht(x), x @ scipy.linalg.hadamard(d) / math.sqrt(d), atol=1e-12)


def test_norm_preserved_and_unit_vector_spread():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((100, 128)) * np.exp(rng.standard_normal(128))
    np.testing.assert_allclose(np.linalg.norm(fwht(x), axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    e0 = np.zeros(128)
    e0[0] = 1
    np.testing.assert_allclose(fwht(e0), np.full(128, 1 / math.sqrt(128)), atol=1e-15)
    # fp32 arithmetic keeps the norm to ~1e-6 relative as well
    x32 = x.astype(np.float32)
    y32 = fwht(x32).astype(np.float32)
    np.testing.assert_allclose(np.linalg.norm(y32, axis=1), np.linalg.norm(x32.astype(np.float64), axis=1), rtol=1e-6)
