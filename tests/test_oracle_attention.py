"""Pins of the oracle's attention over the compressed, paged cache."""
import math

import numpy as np
import scipy.special
import pytest
import torch

from oracle import (attention_dense, codebook_fp32, decode_paged, decode_paged_hot, dequant_k, dequant_v,
                    encode_k, encode_v, fwht, gaussian_matrix)
from oracle.pages import K_PAGE_BYTES, V_PAGE_BYTES, write_slots_fast
from oracle.qjl import qjl_alpha


def _sdpa(q, k, v, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=scale)
    return out[0, 0, 0].numpy()


def test_dense_attention_is_library_softmax_attention():
    rng = np.random.default_rng(0)
    for L in (1, 5, 300):
        q = rng.standard_normal(16)
        k = rng.standard_normal((L, 16)) * 3
        v = rng.standard_normal((L, 16))
        np.testing.assert_allclose(attention_dense(q, k, v, 0.25), _sdpa(q, k, v, 0.25), rtol=1e-12, atol=1e-13)
    assert np.all(attention_dense(q, k[:0], v[:0], 1.0) == 0)


@pytest.mark.parametrize("d", [4, 8, 16, 128])
def test_rotated_domain_form_equals_definition(d):
    # The fast form scores with H q and S q, accumulates codebook values in
    # the rotated domain and applies one inverse rotation at the end.  It
    # must equal the explicit definition up to rounding.
    rng = np.random.default_rng(d)
    c32, t32 = codebook_fp32(d, 3)
    S = rng.standard_normal((d, d)).astype(np.float32)
    L = 8 if d < 128 else 200
    x = rng.standard_normal((L, d)) * 4
    xv = rng.standard_normal((L, d)) * 2
    q = rng.standard_normal(d)
    ek = encode_k(x, c32, t32, S)
    ev = encode_v(xv, c32, t32)
    scale = 1 / math.sqrt(d)
    ref = attention_dense(q, dequant_k(ek["codes"], ek["signs"], ek["norm_f16"], ek["gamma_f16"], c32, S),
                          dequant_v(ev["codes"], ev["norm_f16"], c32), scale)
    c = c32.astype(np.float64)
    qr = fwht(q)
    s = S.astype(np.float64) @ q
    sig = 2.0 * ek["signs"] - 1.0
    nk = ek["norm_f16"].astype(np.float64)
    gk = ek["gamma_f16"].astype(np.float64)
    sc = scale * nk * (c[ek["codes"].astype(int)] @ qr + qjl_alpha(d) * gk * (sig @ s))
    p = np.exp(sc - sc.max())
    acc = (p * ev["norm_f16"].astype(np.float64)) @ c[ev["codes"].astype(int)]
    fast = fwht(acc / p.sum())
    np.testing.assert_allclose(fast, ref, rtol=1e-11, atol=1e-12)


def _pool(rng, T, Hkv, c32, t32, S, x=None, xv=None):
    nb = (T + 15) // 16
    x = rng.standard_normal((T, Hkv, 128)) * 3 if x is None else x
    xv = rng.standard_normal((T, Hkv, 128)) if xv is None else xv
    ek = encode_k(x, c32, t32, S)
    ev = encode_v(xv, c32, t32)
    kp = np.zeros((nb, Hkv, K_PAGE_BYTES), np.uint8)
    vp = np.zeros((nb, Hkv, V_PAGE_BYTES), np.uint8)
    perm = rng.permutation(nb)
    slots = perm[np.arange(T) // 16] * 16 + np.arange(T) % 16
    write_slots_fast(kp, vp, slots, ek, ev)
    return kp, vp, perm[None].astype(np.int32), ek, ev


def test_paged_special_cases():
    rng = np.random.default_rng(1)
    c32, t32 = codebook_fp32()
    S = gaussian_matrix(42)
    kp, vp, table, ek, ev = _pool(rng, 40, 2, c32, t32, S)
    q = rng.standard_normal((1, 1, 4, 128))
    vals = [dequant_v(ev["codes"][:, h], ev["norm_f16"][:, h], c32) for h in range(2)]
    # one visible token -> its value
    o = decode_paged(q, kp, vp, table, np.array([1]), c32, S)
    for hq in range(4):
        np.testing.assert_allclose(o[0, 0, hq], vals[hq // 2][0], rtol=1e-12)
    # zero query -> plain mean of the values
    o = decode_paged(np.zeros_like(q), kp, vp, table, np.array([40]), c32, S)
    for hq in range(4):
        np.testing.assert_allclose(o[0, 0, hq], vals[hq // 2].mean(axis=0), rtol=1e-12, atol=1e-14)
    # empty context -> zeros
    o = decode_paged(q, kp, vp, table, np.array([0]), c32, S)
    assert np.all(o == 0)


def test_without_qjl_term_is_softmax_attention_on_rotated_back_levels():
    rng = np.random.default_rng(2)
    c32, t32 = codebook_fp32()
    S = gaussian_matrix(42)
    T = 50
    x = rng.standard_normal((T, 1, 128)) * 3
    kp, vp, table, ek, ev = _pool(rng, T, 1, c32, t32, S, x=x)
    # force every gamma to +0.0 in the pool
    kp[:, :, 1056:1088] = 0
    q = rng.standard_normal((1, 1, 1, 128))
    o = decode_paged(q, kp, vp, table, np.array([T]), c32, S)
    keys = ek["norm_f16"][:, 0, None].astype(np.float64) * fwht(c32.astype(np.float64)[ek["codes"][:, 0].astype(int)])
    vals = ev["norm_f16"][:, 0, None].astype(np.float64) * fwht(c32.astype(np.float64)[ev["codes"][:, 0].astype(int)])
    np.testing.assert_allclose(o[0, 0, 0], _sdpa(q[0, 0, 0], keys, vals, 1 / math.sqrt(128)), rtol=1e-11)


def test_block_table_permutation_and_gqa_mapping():
    rng = np.random.default_rng(3)
    c32, t32 = codebook_fp32()
    S = gaussian_matrix(42)
    T, Hkv = 70, 2
    kp, vp, table, ek, ev = _pool(rng, T, Hkv, c32, t32, S)
    q = rng.standard_normal((1, 1, 8, 128))
    o1 = decode_paged(q, kp, vp, table, np.array([T]), c32, S)
    # relabel the physical blocks: same logical content, same answer
    nb = kp.shape[0]
    relabel = rng.permutation(nb)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[relabel] = kp
    vp2[relabel] = vp
    o2 = decode_paged(q, kp2, vp2, relabel[table], np.array([T]), c32, S)
    np.testing.assert_array_equal(o1, o2)
    # q-heads 0..3 read KV head 0, 4..7 read KV head 1
    for hq in range(8):
        h = hq // 4
        keys = dequant_k(ek["codes"][:, h], ek["signs"][:, h], ek["norm_f16"][:, h], ek["gamma_f16"][:, h], c32, S)
        vals = dequant_v(ev["codes"][:, h], ev["norm_f16"][:, h], c32)
        np.testing.assert_allclose(o1[0, 0, hq], attention_dense(q[0, 0, hq], keys, vals, 1 / math.sqrt(128)), rtol=1e-12)


def test_causal_rows_equal_single_query_calls():
    rng = np.random.default_rng(4)
    c32, t32 = codebook_fp32()
    S = gaussian_matrix(42)
    T, q_len = 45, 6
    kp, vp, table, _, _ = _pool(rng, T, 1, c32, t32, S)
    q = rng.standard_normal((1, q_len, 2, 128))
    o = decode_paged(q, kp, vp, table, np.array([T]), c32, S)
    for t in range(q_len):
        single = decode_paged(q[:, t:t + 1], kp, vp, table, np.array([T - q_len + t + 1]), c32, S)
        np.testing.assert_array_equal(o[:, t], single[:, 0])
    # the rows differ: each sees one more key than the previous
    assert not np.allclose(o[0, 0], o[0, 1])


def test_hot_window_pins():
    # Compressed history followed by an exact hot window in one softmax.
    rng = np.random.default_rng(5)
    c32, t32 = codebook_fp32()
    S = gaussian_matrix(42)
    T, Hkv, G, W = 60, 2, 3, 9
    kp, vp, table, ek, ev = _pool(rng, T, Hkv, c32, t32, S)
    hk = (rng.standard_normal((1, W, Hkv, 128)) * 3).astype(np.float32)
    hv = rng.standard_normal((1, W, Hkv, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, G * Hkv, 128))
    scale = 1 / math.sqrt(128)
    # no window: the compressed-cache attention itself
    np.testing.assert_array_equal(decode_paged_hot(q, kp, vp, table, np.array([T]), hk, hv, np.array([0]), c32, S),
                                  decode_paged(q, kp, vp, table, np.array([T]), c32, S))
    # no history: library softmax attention on the exact window
    o = decode_paged_hot(q, kp, vp, table, np.array([0]), hk, hv, np.array([W]), c32, S)
    for hq in range(G * Hkv):
        h = hq // G
        np.testing.assert_allclose(o[0, 0, hq], _sdpa(q[0, 0, hq], hk[0, :, h].astype(np.float64),
                                                      hv[0, :, h].astype(np.float64), scale), rtol=1e-12, atol=1e-13)
    # both: the log-sum-exp combination of the two partitions' attentions
    L, Wb = 37, 5
    o = decode_paged_hot(q, kp, vp, table, np.array([L]), hk, hv, np.array([Wb]), c32, S)
    for hq in range(G * Hkv):
        h = hq // G
        kc = dequant_k(ek["codes"][:L, h], ek["signs"][:L, h], ek["norm_f16"][:L, h], ek["gamma_f16"][:L, h], c32, S)
        vc = dequant_v(ev["codes"][:L, h], ev["norm_f16"][:L, h], c32)
        kh, vh = hk[0, :Wb, h].astype(np.float64), hv[0, :Wb, h].astype(np.float64)
        lse_c = scipy.special.logsumexp(scale * (kc @ q[0, 0, hq]))
        lse_h = scipy.special.logsumexp(scale * (kh @ q[0, 0, hq]))
        wc = 1.0 / (1.0 + math.exp(lse_h - lse_c))
        ref = wc * _sdpa(q[0, 0, hq], kc, vc, scale) + (1.0 - wc) * _sdpa(q[0, 0, hq], kh, vh, scale)
        np.testing.assert_allclose(o[0, 0, hq], ref, rtol=1e-10, atol=1e-12)
    # several new tokens at the end of the window: causal inside it, the last
    # one equals the single-query call
    q3 = rng.standard_normal((1, 3, G * Hkv, 128))
    o3 = decode_paged_hot(q3, kp, vp, table, np.array([L]), hk, hv, np.array([Wb]), c32, S)
    for t in range(3):
        single = decode_paged_hot(q3[:, t:t + 1], kp, vp, table, np.array([L]), hk, hv, np.array([Wb - 2 + t]), c32, S)
        np.testing.assert_array_equal(o3[:, t], single[:, 0])


def _sphere_coordinate_distortion(c32, t32, d):
    """d * E[(y - Q(y))^2] for one coordinate y of a point drawn uniformly on
    the unit sphere in R^d (density proportional to (1 - y^2)^((d-3)/2) on
    [-1, 1]), by adaptive quadrature over the cells of the fp32 codebook."""
    from scipy import integrate, special
    c = np.asarray(c32, np.float64)
    t = np.asarray(t32, np.float64)
    log_c = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)

    def dens(y):
        return math.exp(log_c + 0.5 * (d - 3) * math.log1p(-y * y))

    edges = [-1.0, *t, 1.0]
    total = 0.0
    for k in range(len(c)):
        total += integrate.quad(lambda y: (y - c[k]) ** 2 * dens(y), edges[k], edges[k + 1],
                                epsabs=1e-14, epsrel=1e-12)[0]
    return d * total


def test_dequant_v_reconstruction_error_is_the_codebook_distortion():
    # For an isotropic x, u = x/|x| is uniform on the sphere and so is y = H u
    # (H orthogonal); dequant_v(encode_v(x)) = n H^T c[idx] differs from x by
    # n H^T (c[idx] - y), so |x^ - x|^2 / |x|^2 = |y - c[idx]|^2 up to the
    # half rounding of n.  Its mean is the quantiser's distortion on the
    # sphere marginal, computed here by quadrature, and close to Max's
    # Gaussian figure 0.03454 (the sphere marginal has lighter tails).
    # With the centroid condition E<c[idx], y> = E|c[idx]|^2 = 1 - D, so the
    # cosine between x^ and x is about sqrt(1 - D).
    rng = np.random.default_rng(21)
    c32, t32 = codebook_fp32(128, 3)
    n = 20000
    x = rng.standard_normal((n, 128)) * rng.exponential(5.0, (n, 1))
    ev = encode_v(x, c32, t32)
    xh = dequant_v(ev["codes"], ev["norm_f16"], c32)
    rel = np.sum((xh - x) ** 2, axis=-1) / np.sum(x * x, axis=-1)
    D = _sphere_coordinate_distortion(c32, t32, 128)
    se = rel.std(ddof=1) / math.sqrt(n)
    assert abs(rel.mean() - D) < 4 * se + 1e-6, (rel.mean(), D, se)
    assert abs(D / 0.03454 - 1.0) < 0.03
    cos = np.sum(xh * x, axis=-1) / (np.linalg.norm(xh, axis=-1) * np.linalg.norm(x, axis=-1))
    assert abs(cos.mean() - math.sqrt(1.0 - D)) < 5e-4, (cos.mean(), math.sqrt(1.0 - D))


def test_dequant_v_closed_forms():
    # Every code at the top level: c[7] * (1, ..., 1) rotates back to
    # c[7] sqrt(d) e_0 (the first Sylvester row is the only one with a
    # non-zero sum).  Codes following the sign pattern of Sylvester row j
    # (7 where the entry is positive, 0 where negative; c[0] = -c[7]) rotate
    # back to c[7] sqrt(d) e_j.  The stored half norm multiplies the result.
    c32, _ = codebook_fp32(128, 3)
    c7 = float(c32[7])
    assert c32[0] == -c32[7]
    n16 = np.array([3.5], dtype=np.float16)
    out = dequant_v(np.full((1, 128), 7, np.uint8), n16, c32)[0]
    want = np.zeros(128)
    want[0] = 3.5 * c7 * math.sqrt(128)
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13)
    hrow = np.ones((1, 1))
    while hrow.shape[0] < 128:
        hrow = np.block([[hrow, hrow], [hrow, -hrow]])
    for j in (1, 37, 127):
        codes = np.where(hrow[j] > 0, 7, 0).astype(np.uint8)[None]
        out = dequant_v(codes, np.array([2.0], np.float16), c32)[0]
        want = np.zeros(128)
        want[j] = 2.0 * c7 * math.sqrt(128)
        np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13)
