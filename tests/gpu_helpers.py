"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle at the tolerances the method's contract states:
codes and sign bits bit-exact except within 1e-5 of a decision threshold,
norms to 1e-6 relative, attention outputs to 2e-3 relative: per row, both
the L2 error against the row's L2 norm and every coordinate's error against
the row's largest magnitude."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_tq_amd as tq
from oracle import codebook_fp32, decode_paged, encode_k, encode_v, gaussian_matrix
from oracle.encode import residual_signs_from_codes
from oracle.pages import k_page_bytes, read_k_tokens_fast, read_v_tokens_fast, v_page_bytes

CODE_BAND = 1e-5
SIGN_BAND = 1e-5
NORM_RTOL = 1e-6
OUT_RTOL = 2e-3
QJL_SEED = 42

_CB = {}


def codebook(seed: int = QJL_SEED, bits: int = 3):
    if (seed, bits) not in _CB:
        _CB[(seed, bits)] = tq.tq_codebook_init(128, bits, seed, device="cuda")
    return _CB[(seed, bits)]


def oracle_tables(seed: int = QJL_SEED, bits: int = 3):
    c32, t32 = codebook_fp32(128, bits)
    return c32, t32, gaussian_matrix(seed, 128, 128)


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def new_pools(num_blocks: int, Hkv: int, fill: str = "random", seed: int = 0, bits: int = 3):
    kb, vb = k_page_bytes(bits), v_page_bytes(bits)
    if fill == "random":
        g = torch.Generator(device="cpu").manual_seed(seed)
        k = torch.randint(0, 256, (num_blocks, Hkv, kb), dtype=torch.uint8, generator=g)
        v = torch.randint(0, 256, (num_blocks, Hkv, vb), dtype=torch.uint8, generator=g)
        return k.cuda(), v.cuda()
    return (torch.zeros((num_blocks, Hkv, kb), dtype=torch.uint8, device="cuda"),
            torch.zeros((num_blocks, Hkv, vb), dtype=torch.uint8, device="cuda"))


def encode_gpu(cb, k, v, slots, kpool, vpool, dtype=torch.bfloat16, with_norms=True):
    kt, vt = dev(k, dtype), dev(v, dtype)
    st = torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda()
    norms = None
    if with_norms:
        norms = torch.full((k.shape[0], k.shape[1], 3), float("nan"), device="cuda")
    tq.tq_encode_kv(cb, kt, vt, st, kpool, vpool, norms)
    torch.cuda.synchronize()
    return None if norms is None else norms.cpu().numpy()


def _near_threshold(y, t32):
    return np.min(np.abs(np.asarray(y)[..., None] - t32.astype(np.float64)), axis=-1) < CODE_BAND


def _half_ok(stored, exact):
    """Stored half equals round-to-nearest-even of the exact value, allowing the
    other neighbour only when the exact value is within 1e-6 of a midpoint."""
    exact = np.asarray(exact, dtype=np.float64)
    lo = np.minimum(exact * (1 - NORM_RTOL), 65504.0).astype(np.float16)
    hi = np.minimum(exact * (1 + NORM_RTOL), 65504.0).astype(np.float16)
    return (stored == lo) | (stored == hi)


def check_encoded_sequence(k, v, kpool_np, vpool_np, table_row, positions, norms,
                           tables=None, stats=None):
    """Compare the GPU records of tokens ``positions`` (their keys/values are
    ``k[j]``, ``v[j]``, shape [n][Hkv][128]) of one sequence against the
    oracle.  ``norms`` is the GPU's fp32 (|k|, gamma, |v|) per token/head or None."""
    c32, t32, S = tables or oracle_tables()
    positions = np.asarray(positions)
    Hkv = k.shape[1]
    L = int(positions.max()) + 1
    ek = encode_k(k, c32, t32, S)
    ev = encode_v(v, c32, t32)
    for h in range(Hkv):
        kc, ks, kn, kg = read_k_tokens_fast(kpool_np, table_row, L, h)
        vc, vn = read_v_tokens_fast(vpool_np, table_row, L, h)
        kc, ks, kn, kg, vc, vn = (a[positions] for a in (kc, ks, kn, kg, vc, vn))
        # codes: bit-exact away from thresholds
        amb_k = _near_threshold(ek["y"][:, h], t32)
        amb_v = _near_threshold(ev["y"][:, h], t32)
        bad_k = (kc != ek["codes"][:, h]) & ~amb_k
        bad_v = (vc != ev["codes"][:, h]) & ~amb_v
        assert not bad_k.any(), f"head {h}: {int(bad_k.sum())} key codes differ outside the band"
        assert not bad_v.any(), f"head {h}: {int(bad_v.sum())} value codes differ outside the band"
        # sign bits: oracle signs recomputed from the GPU's codes
        gam, z, bits = residual_signs_from_codes(k[:, h], kc, c32, S)
        bad_s = (ks != bits) & (np.abs(z) >= SIGN_BAND)
        assert not bad_s.any(), f"head {h}: {int(bad_s.sum())} sign bits differ outside the band"
        # stored half scalars
        assert _half_ok(kn, ek["norm"][:, h]).all(), f"head {h}: key norm halves"
        assert _half_ok(kg, gam).all(), f"head {h}: gamma halves"
        assert _half_ok(vn, ev["norm"][:, h]).all(), f"head {h}: value norm halves"
        if norms is not None:
            np.testing.assert_allclose(norms[:, h, 0], ek["norm"][:, h], rtol=NORM_RTOL, atol=1e-30)
            np.testing.assert_allclose(norms[:, h, 1], gam, rtol=NORM_RTOL, atol=1e-7)
            np.testing.assert_allclose(norms[:, h, 2], ev["norm"][:, h], rtol=NORM_RTOL, atol=1e-30)
        if stats is not None:
            stats["ambiguous_codes"] = stats.get("ambiguous_codes", 0) + int(amb_k.sum() + amb_v.sum())
            stats["code_mismatch_in_band"] = stats.get("code_mismatch_in_band", 0) + int(
                ((kc != ek["codes"][:, h]) & amb_k).sum() + ((vc != ev["codes"][:, h]) & amb_v).sum())
            stats["coords"] = stats.get("coords", 0) + 2 * kc.size


def decode_gpu(cb, q, kpool, vpool, table, context_lens, Hkv, q_dtype=torch.bfloat16,
               out_dtype=torch.float32, tokens_per_split=0, scale=0.0):
    qt = dev(q, q_dtype)
    bt = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    cl = torch.from_numpy(np.ascontiguousarray(context_lens, dtype=np.int32)).cuda()
    out = tq.tq_decode_attention(cb, qt, kpool, vpool, bt, cl, int(max(context_lens.max(), 0)),
                                 Hkv, softmax_scale=scale, tokens_per_split=tokens_per_split,
                                 out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def rel_rows(out, ref):
    """Per-row relative L2 error over the rows the reference computed."""
    mask = ~np.isnan(ref[..., 0])
    o = out[mask].astype(np.float64)
    r = ref[mask]
    num = np.linalg.norm(o - r, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def elementwise_rows(out, ref):
    """Per row, the largest coordinate error over the row's largest reference
    magnitude (rows the reference computed)."""
    mask = ~np.isnan(ref[..., 0])
    o = out[mask].astype(np.float64)
    r = ref[mask]
    num = np.max(np.abs(o - r), axis=-1)
    den = np.max(np.abs(r), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def assert_rows_close(out, ref, rtol=OUT_RTOL):
    """Both bars: per-row relative L2 and per-coordinate error against the
    row's largest magnitude, each at ``rtol``; reports the worst row."""
    err = rel_rows(out, ref)
    ew = elementwise_rows(out, ref)
    assert err.size > 0
    mask = ~np.isnan(ref[..., 0])
    idx = np.argwhere(mask)
    assert err.max() <= rtol, f"max row rel L2 err {err.max():.3e} > {rtol} at row {idx[int(err.argmax())]}"
    assert ew.max() <= rtol, (f"max coordinate err / row max {ew.max():.3e} > {rtol} "
                              f"at row {idx[int(ew.argmax())]}")
    return err


def check_decode(out, q, kpool_np, vpool_np, table, context_lens, tables=None, rtol=OUT_RTOL,
                 scale=None, **subset):
    c32, _, S = tables or oracle_tables()
    q64 = np.asarray(q, dtype=np.float64)
    ref = decode_paged(q64, kpool_np, vpool_np, table, context_lens, c32, S, scale=scale, **subset)
    return assert_rows_close(out, ref, rtol)
