"""Attention read from the compressed cache, by its plain definition (float64).

The pages say attention runs over the whole compressed history ([C] the
note on ``--turbo-kv`` long-range recall) with dequantisation fused into the
GPU kernel ([A] "TurboQuant V2+V3ハイブリッド実装"), and that the V cache
carries no QJL term because values are not used in the score inner product
([C] V-cache paragraph).  The oracle does not use any rotated-domain or
fused trick: it rebuilds every key and value explicitly and applies
softmax(scale * q.k) v.

Readings taken where the pages are silent:
  * Dequantised value:  v~ = n_v * H^T c[idx_v]  (no re-normalisation).
  * Dequantised key, with the QJL estimator of <q, r> (see qjl.py):
        k~ = n_k * (H^T c[idx_k] + alpha * gamma * S^T sigma),
    sigma_i = 2*bit_i - 1, alpha = sqrt(pi/2)/m, so that <q, k~> equals
    n_k * (<q, H^T yhat> + estimate of <q, r>).  n_k, gamma, n_v are the
    stored half values.
  * GQA: query head h reads KV head h // (Hq / Hkv).
  * More than one query per sequence (chunked prefill) is causal: query t
    of q_len sees keys 0 .. L - q_len + t, L the context length including
    the new tokens.  An empty visible range gives a zero output.
  * Softmax scale 1/sqrt(d) unless given.
  * Hot window (decode_paged_hot): the pages compress the cache only past a
    threshold and keep the recent tokens uncompressed ([C] the --turbo-kv
    option row of the server options table: compression starts after 2,048
    tokens), and attention covers the compressed history as well as that
    window ([C] the note on --turbo-kv long-range recall).  Sequence b holds
    its first L_b tokens compressed and the next W_b tokens exactly; the
    softmax runs over all L_b + W_b keys.  The q_len new tokens are the last
    q_len of the window, and query t sees the whole history and window
    tokens 0 .. W_b - q_len + t.
"""

from __future__ import annotations

import math

import numpy as np

from .hadamard import sylvester_hadamard
from .pages import BLOCK, read_k_tokens_fast, read_v_tokens_fast
from .qjl import qjl_alpha


def dequant_v(codes, n16, centroids_f32) -> np.ndarray:
    codes = np.asarray(codes)
    d = codes.shape[-1]
    c = np.asarray(centroids_f32, dtype=np.float32).astype(np.float64)
    yhat = c[codes.astype(np.int64)]
    n = np.asarray(n16, dtype=np.float16).astype(np.float64)
    return n[..., None] * (yhat @ sylvester_hadamard(d))


def dequant_k(codes, signs, n16, g16, centroids_f32, S_f32) -> np.ndarray:
    codes = np.asarray(codes)
    d = codes.shape[-1]
    S = np.asarray(S_f32, dtype=np.float32).astype(np.float64)
    m = S.shape[0]
    c = np.asarray(centroids_f32, dtype=np.float32).astype(np.float64)
    yhat = c[codes.astype(np.int64)]
    sigma = 2.0 * np.asarray(signs, dtype=np.float64) - 1.0
    n = np.asarray(n16, dtype=np.float16).astype(np.float64)
    g = np.asarray(g16, dtype=np.float16).astype(np.float64)
    corr = qjl_alpha(m) * g[..., None] * (sigma @ S)          # S^T sigma as a row
    return n[..., None] * (yhat @ sylvester_hadamard(d) + corr)


def attention_dense(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                    scale: float) -> np.ndarray:
    """softmax(scale * keys @ q) @ values for one query ``q[d]``."""
    q = np.asarray(q, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64)
    s = scale * (keys @ q)
    w = np.exp(s - np.max(s))
    return (w / np.sum(w)) @ values


def decode_paged(q, k_pool, v_pool, block_tables, context_lens, centroids_f32, S_f32,
                 scale: float | None = None, kv_heads=None, seqs=None,
                 q_positions=None) -> np.ndarray:
    """Attention of ``q[B][q_len][Hq][d]`` over the paged compressed cache.

    Returns float64 ``[B][q_len][Hq][d]``; rows outside the optional
    ``seqs`` / ``kv_heads`` / ``q_positions`` subsets are left as NaN so a
    caller checking a sample cannot mistake them for results.
    """
    q = np.asarray(q, dtype=np.float64)
    B, q_len, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    out = np.full(q.shape, np.nan)
    seqs = range(B) if seqs is None else seqs
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    q_positions = range(q_len) if q_positions is None else q_positions
    for b in seqs:
        L = int(context_lens[b])
        row = block_tables[b]
        for h in kv_heads:
            kc, ks, kn, kg = read_k_tokens_fast(k_pool, row, L, h)
            vc, vn = read_v_tokens_fast(v_pool, row, L, h)
            keys = dequant_k(kc, ks, kn, kg, centroids_f32, S_f32)
            vals = dequant_v(vc, vn, centroids_f32)
            for t in q_positions:
                vis = max(0, L - q_len + t + 1)
                for g in range(G):
                    hq = h * G + g
                    out[b, t, hq] = attention_dense(q[b, t, hq], keys[:vis], vals[:vis], scale)
    return out


def decode_paged_hot(q, k_pool, v_pool, block_tables, context_lens, hot_k, hot_v, hot_lens,
                     centroids_f32, S_f32, scale: float | None = None, kv_heads=None,
                     seqs=None) -> np.ndarray:
    """Attention of ``q[B][q_len][Hq][d]`` over the compressed history of
    ``context_lens[b]`` tokens followed by ``hot_lens[b]`` exact tokens
    ``hot_k[b][j][h]``, ``hot_v[b][j][h]`` (any float dtype, taken exactly).

    Returns float64 ``[B][q_len][Hq][d]``; rows outside the optional subsets
    are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, q_len, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    out = np.full(q.shape, np.nan)
    seqs = range(B) if seqs is None else seqs
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    for b in seqs:
        L, W = int(context_lens[b]), int(hot_lens[b])
        row = block_tables[b]
        for h in kv_heads:
            kc, ks, kn, kg = read_k_tokens_fast(k_pool, row, L, h)
            vc, vn = read_v_tokens_fast(v_pool, row, L, h)
            keys = np.concatenate([dequant_k(kc, ks, kn, kg, centroids_f32, S_f32),
                                   np.asarray(hot_k[b, :W, h], dtype=np.float64)])
            vals = np.concatenate([dequant_v(vc, vn, centroids_f32),
                                   np.asarray(hot_v[b, :W, h], dtype=np.float64)])
            for t in range(q_len):
                vis = L + max(0, W - q_len + t + 1)
                for g in range(G):
                    hq = h * G + g
                    out[b, t, hq] = attention_dense(q[b, t, hq], keys[:vis], vals[:vis], scale)
    return out


def ring_row(block_row, length: int) -> np.ndarray:
    """Block-table entries of logical pages 0 .. ceil(length / 16) - 1 when
    the row is a ring of ``len(block_row)`` pages: page P sits in entry
    P mod len(block_row), so a page is reused for the positions 16 R later."""
    row = np.asarray(block_row)
    nb = (length + BLOCK - 1) // BLOCK
    return row[np.arange(nb) % len(row)]


def decode_paged_window(q, k_pool, v_pool, block_tables, context_lens, window: int,
                        centroids_f32, S_f32, scale: float | None = None, kv_heads=None,
                        seqs=None, q_positions=None) -> np.ndarray:
    """Sliding-window attention of ``q[B][q_len][Hq][d]`` over a rotating
    paged cache.

    The SwiftLM README ("Performance: Mac mini M6", the correction under its
    tables and the --turbo-kv recall note) says sliding-window layers run on
    a rotating cache (Gemma 4: 1,024-token window on 25 of 30 layers) that
    keeps only the most recent tokens.  Reading taken: query t of sequence b
    sits at position p = L - q_len + t and attends to the keys at positions
    max(0, p - window + 1) .. p (its own and the window - 1 before it); the
    cache keeps them in a ring of R = len(block_tables[b]) pages, position j
    in page ``block_tables[b][(j // 16) mod R]`` at offset j % 16.

    Returns float64 ``[B][q_len][Hq][d]``; rows outside the optional subsets
    are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, q_len, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    out = np.full(q.shape, np.nan)
    seqs = range(B) if seqs is None else seqs
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    q_positions = range(q_len) if q_positions is None else q_positions
    for b in seqs:
        L = int(context_lens[b])
        row = ring_row(block_tables[b], L)
        for h in kv_heads:
            kc, ks, kn, kg = read_k_tokens_fast(k_pool, row, L, h)
            vc, vn = read_v_tokens_fast(v_pool, row, L, h)
            keys = dequant_k(kc, ks, kn, kg, centroids_f32, S_f32)
            vals = dequant_v(vc, vn, centroids_f32)
            for t in q_positions:
                hi = max(0, L - q_len + t + 1)
                lo = max(0, hi - window)
                for g in range(G):
                    hq = h * G + g
                    out[b, t, hq] = attention_dense(q[b, t, hq], keys[lo:hi], vals[lo:hi], scale)
    return out

