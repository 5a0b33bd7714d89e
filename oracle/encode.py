"""TurboQuant encoding of key and value vectors (plain definition, float64).

Key path, in the order of [C] "TurboQuantization: KV Cache Compression",
K-cache steps 1-5 (same list in [A] "KVキャッシュ圧縮の内訳"):
  1. n = ||x||_2 and u = x / n;
  2. y = H u (orthonormal Walsh-Hadamard rotation);
  3. idx_i = index of the Lloyd-Max cell holding y_i, yhat_i = c[idx_i];
  4. residual between the normalised original and its quantised
     approximation, r = u - H^T yhat, and its length gamma = ||r||;
  5. z = S r and one sign bit per row, bit_i = [z_i >= 0].
Value path ([C] V-cache paragraph): steps 1-3 only.

Readings taken where the pages are silent:
  * Zero vector: n = 0 gives u = 0 (no division).
  * Cell search: idx_i = #{j : t_j < y_i}, so a value equal to a threshold
    goes to the lower cell.  The comparison is made in float32 (y rounded
    once from float64), the precision of the float32 codebook.
  * Stored scalars: n and gamma are kept as IEEE half, round-to-nearest-even
    from float64, saturating at 65504 (larger norms are out of contract).
  * Residual domain: the normalised original domain, r = u - H^T yhat, as the
    pages word it; the decoder therefore projects the unrotated query, S q.
"""

from __future__ import annotations

import numpy as np

from .hadamard import sylvester_hadamard

F16_MAX = 65504.0


def to_half_saturating(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return np.minimum(v, F16_MAX).astype(np.float16)


def quantize_codes(y: np.ndarray, thresholds_f32: np.ndarray) -> np.ndarray:
    """idx = #{j : t_j < y} per coordinate, compared in float32."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    t = np.asarray(thresholds_f32, dtype=np.float32)
    idx = np.zeros(y32.shape, dtype=np.int64)
    for tj in t:
        idx += (tj < y32)
    return idx.astype(np.uint8)


def _normalise(x: np.ndarray):
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(n > 0.0, n, 1.0)
    u = np.where(n[..., None] > 0.0, x / safe[..., None], 0.0)
    return n, u


def encode_v(x: np.ndarray, centroids_f32, thresholds_f32) -> dict:
    """Value path for a batch ``x[..., d]``: returns codes, norm (float64 and
    stored half) and the rotated vector y."""
    n, u = _normalise(x)
    d = u.shape[-1]
    h = sylvester_hadamard(d)
    y = u @ h                                   # H symmetric: row-vector form of H u
    idx = quantize_codes(y, thresholds_f32)
    return {"codes": idx, "norm": n, "norm_f16": to_half_saturating(n), "y": y}


def encode_k(x: np.ndarray, centroids_f32, thresholds_f32, S_f32) -> dict:
    """Key path for a batch ``x[..., d]`` with QJL matrix ``S_f32`` (m x d)."""
    out = encode_v(x, centroids_f32, thresholds_f32)
    d = out["y"].shape[-1]
    h = sylvester_hadamard(d)
    c = np.asarray(centroids_f32, dtype=np.float32).astype(np.float64)
    yhat = c[out["codes"].astype(np.int64)]
    n, u = _normalise(x)
    r = u - yhat @ h                            # step 4, original domain
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    S = np.asarray(S_f32, dtype=np.float32).astype(np.float64)
    z = r @ S.T                                 # step 5: z_i = sum_k S[i, k] r_k
    bits = (z >= 0.0).astype(np.uint8)
    out.update({"signs": bits, "z": z, "gamma": gamma,
                "gamma_f16": to_half_saturating(gamma), "residual": r})
    return out


def residual_signs_from_codes(x: np.ndarray, codes: np.ndarray, centroids_f32,
                              S_f32):
    """Steps 4-5 for given codes: (gamma, z, bits).  Used to check sign bits
    against codes produced elsewhere, since one flipped code changes the whole
    residual."""
    n, u = _normalise(x)
    d = u.shape[-1]
    h = sylvester_hadamard(d)
    c = np.asarray(centroids_f32, dtype=np.float32).astype(np.float64)
    r = u - c[np.asarray(codes).astype(np.int64)] @ h
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    z = r @ np.asarray(S_f32, dtype=np.float32).astype(np.float64).T
    return gamma, z, (z >= 0.0).astype(np.uint8)
