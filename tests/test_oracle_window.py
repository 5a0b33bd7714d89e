"""Pins of the oracle's sliding-window attention over a rotating cache.

The expected values are built without the oracle's page reader: from the
encodings themselves (encode_k / encode_v) of the keys each query must see,
so that a wrong ring index, a window off by one or a wrong causal end fails."""
import numpy as np
import pytest

from oracle import (attention_dense, codebook_fp32, decode_paged, decode_paged_window, dequant_k, dequant_v,
                    encode_k, encode_v, gaussian_matrix, ring_row)
from oracle.pages import K_PAGE_BYTES, V_PAGE_BYTES, write_slots

D = 128


def _tables():
    c32, t32 = codebook_fp32(D, 3)
    return c32, t32, gaussian_matrix(42).astype(np.float32)


def _ring_cache(rng, N, Hkv, R, pool_blocks, c32, t32, S):
    """N tokens written in position order into a ring of R pages (older
    positions overwritten), with their encodings kept aside."""
    row = rng.permutation(pool_blocks)[:R].astype(np.int32)
    x = rng.standard_normal((N, Hkv, D)) * rng.uniform(0.5, 3.0, (N, Hkv, 1))
    y = rng.standard_normal((N, Hkv, D))
    ek, ev = encode_k(x, c32, t32, S), encode_v(y, c32, t32)
    kp = np.zeros((pool_blocks, Hkv, K_PAGE_BYTES), np.uint8)
    vp = np.zeros((pool_blocks, Hkv, V_PAGE_BYTES), np.uint8)
    slots = np.array([row[(j // 16) % R] * 16 + j % 16 for j in range(N)], np.int64)
    write_slots(kp, vp, slots, ek, ev)   # one token at a time, in order
    return row, ek, ev, kp, vp


def test_ring_row_wraps_modulo_the_row_length():
    row = np.array([7, 3, 9])
    assert list(ring_row(row, 16 * 7 + 1)) == [7, 3, 9, 7, 3, 9, 7, 3]
    assert list(ring_row(row, 0)) == []


@pytest.mark.parametrize("N,W,q_len,R", [(100, 30, 3, 3), (77, 77, 1, 5), (200, 48, 1, 3), (64, 17, 5, 2)])
def test_window_attention_is_attention_over_the_last_window_keys(N, W, q_len, R):
    """Query t (position p = N - q_len + t) must equal dense attention over
    the dequantised encodings of positions max(0, p - W + 1) .. p, while the
    pages hold only the last 16 R positions."""
    assert 16 * R >= W + q_len - 1
    rng = np.random.default_rng(N + W)
    c32, t32, S = _tables()
    Hkv, G = 2, 2
    row, ek, ev, kp, vp = _ring_cache(rng, N, Hkv, R, 11, c32, t32, S)
    q = rng.standard_normal((1, q_len, Hkv * G, D))
    out = decode_paged_window(q, kp, vp, row[None, :], np.array([N]), W, c32, S)
    for h in range(Hkv):
        keys = dequant_k(ek["codes"][:, h], ek["signs"][:, h], ek["norm_f16"][:, h], ek["gamma_f16"][:, h], c32, S)
        vals = dequant_v(ev["codes"][:, h], ev["norm_f16"][:, h], c32)
        for t in range(q_len):
            p = N - q_len + t
            lo = max(0, p - W + 1)
            for g in range(G):
                ref = attention_dense(q[0, t, h * G + g], keys[lo:p + 1], vals[lo:p + 1], 1 / np.sqrt(D))
                np.testing.assert_allclose(out[0, t, h * G + g], ref, rtol=1e-12, atol=1e-12)


def test_window_of_one_is_the_own_value():
    """A one-position window leaves each query its own key: the output is
    that token's dequantised value, whatever the query."""
    rng = np.random.default_rng(5)
    c32, t32, S = _tables()
    N, q_len = 90, 4
    row, ek, ev, kp, vp = _ring_cache(rng, N, 1, 2, 6, c32, t32, S)
    q = rng.standard_normal((1, q_len, 1, D)) * 10
    out = decode_paged_window(q, kp, vp, row[None, :], np.array([N]), 1, c32, S)
    vals = dequant_v(ev["codes"][:, 0], ev["norm_f16"][:, 0], c32)
    for t in range(q_len):
        np.testing.assert_allclose(out[0, t, 0], vals[N - q_len + t], rtol=1e-13, atol=1e-13)


def test_window_covering_the_context_is_the_plain_attention():
    """A window at least as long as the context, over a table long enough
    never to wrap, is plain causal attention over the whole cache."""
    rng = np.random.default_rng(6)
    c32, t32, S = _tables()
    N, q_len = 70, 3
    row, ek, ev, kp, vp = _ring_cache(rng, N, 1, 5, 8, c32, t32, S)
    q = rng.standard_normal((1, q_len, 2, D))
    a = decode_paged_window(q, kp, vp, row[None, :], np.array([N]), N, c32, S)
    b = decode_paged(q, kp, vp, row[None, :], np.array([N]), c32, S)
    np.testing.assert_array_equal(a, b)
