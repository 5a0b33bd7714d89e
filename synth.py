"""Seeded synthetic inputs for tests and benchmarks.

This module holds none of the method's arithmetic: it only draws keys,
values, queries, context lengths, block tables and slot mappings.  Both the
CPU oracle and the HIP path are fed from it, so they see identical numbers.

Recipe (the pages measure on real models and prompts that are not available
here; these Gaussian stand-ins have the shapes of the workloads):
  * KV vectors: N(0, 1) per coordinate; "outlier channels" are fixed
    coordinates of one KV head multiplied by 20.  The small single-head case
    uses 4 such channels on plain N(0, 1) fp32 data, the same channels for K
    and V.  The GQA cases use bf16 data with a per-(KV head, channel) scale
    exp(N(0, 1)) (log-normal, sigma = 1) and 2 % of the channels
    (round(0.02 * 128) = 3) as outliers, drawn independently for K and V.
  * Queries: N(0, 1), unscaled.
  * Ragged batches: context lengths floor(exp(U(ln 512, ln 32768))).
  * Block tables: a random permutation of the block pool.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK = 16
HEAD_DIM = 128


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), as fp32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def kv_tensor(rng: np.random.Generator, T: int, Hkv: int, d: int = HEAD_DIM, *,
              outliers: int = 3, lognormal_scale: bool = True,
              outlier_channels=None, bf16: bool = True) -> np.ndarray:
    """[T][Hkv][d] float32 values (bf16-representable when ``bf16``)."""
    x = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    scale = np.ones((Hkv, d), dtype=np.float32)
    if lognormal_scale:
        scale = np.exp(rng.standard_normal((Hkv, d))).astype(np.float32)
    for h in range(Hkv):
        ch = (outlier_channels if outlier_channels is not None
              else rng.choice(d, size=outliers, replace=False))
        scale[h, np.asarray(ch)] *= 20.0
    x = x * scale[None]
    return round_to_bf16(x) if bf16 else x


def kv_tensor_device(seed: int, T: int, Hkv: int, device, d: int = HEAD_DIM, outliers: int = 3):
    """The GQA recipe of ``kv_tensor`` drawn on the device with torch's
    seeded generator (for workloads too large to draw on the host): a bf16
    [T][Hkv][d] tensor, per-(KV head, channel) scale exp(N(0, 1)) and
    ``outliers`` channels x20 per KV head.  Not bit-identical to
    ``kv_tensor``; used for timing only."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    scale = torch.exp(torch.randn((Hkv, d), generator=g, device=device))
    for h in range(Hkv):
        ch = torch.randperm(d, generator=g, device=device)[:outliers]
        scale[h, ch] *= 20.0
    x = torch.randn((T, Hkv, d), generator=g, device=device)
    return (x * scale[None]).to(torch.bfloat16)


def queries(rng: np.random.Generator, B: int, q_len: int, Hq: int, d: int = HEAD_DIM,
            bf16: bool = True) -> np.ndarray:
    q = rng.standard_normal((B, q_len, Hq, d)).astype(np.float32)
    return round_to_bf16(q) if bf16 else q


def ragged_lengths(rng: np.random.Generator, B: int, lo: int = 512, hi: int = 32768) -> np.ndarray:
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    return np.floor(np.exp(u)).astype(np.int64)


def block_tables(rng: np.random.Generator, capacities, extra_blocks: int = 0,
                 shuffle: bool = True):
    """Give sequence b room for ``capacities[b]`` tokens.  Returns
    ``(table[B][max_blocks] int32, num_blocks)``; unused entries are 0."""
    caps = [int(c) for c in capacities]
    need = [(c + BLOCK - 1) // BLOCK for c in caps]
    total = sum(need) + extra_blocks
    perm = rng.permutation(total) if shuffle else np.arange(total)
    width = max(1, max(need) if need else 1)
    table = np.zeros((len(caps), width), dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, total


def slots_for(table: np.ndarray, seq: int, positions) -> np.ndarray:
    """Slot of each token position of sequence ``seq``."""
    pos = np.asarray(positions, dtype=np.int64)
    return table[seq, pos // BLOCK].astype(np.int64) * BLOCK + pos % BLOCK


# ---------------------------------------------------------------------------
# The five workloads.  ``small=True`` shrinks lengths so the oracle finishes
# in seconds while keeping several tiles and a ragged tail.

CONFIGS = {
    1: dict(name="single-head d128 T1024 fp32", B=1, Hq=1, Hkv=1, T=1024),
    2: dict(name="GQA 32q/8kv d128 T8192 bf16", B=1, Hq=32, Hkv=8, T=8192),
    3: dict(name="ragged batch16 GQA 32q/8kv 16-token pages bf16", B=16, Hq=32, Hkv=8),
    4: dict(name="long-context T131072 GQA 32q/4kv split-K bf16", B=1, Hq=32, Hkv=4, T=131072),
    5: dict(name="chunked prefill 2048 new on 32768 cached GQA 32q/8kv bf16", B=1, Hq=32,
            Hkv=8, T=32768, new=2048),
}

QJL_SEED = 42


def single_head_case(seed: int = 1, T: int = 1024):
    """K, V [T][1][128] fp32 with 4 outlier channels shared by K and V, q
    [1][1][1][128] fp32, identity block table."""
    rng = np.random.default_rng(seed)
    ch = rng.choice(HEAD_DIM, size=4, replace=False)
    k = kv_tensor(rng, T, 1, outliers=4, lognormal_scale=False, outlier_channels=ch, bf16=False)
    v = kv_tensor(rng, T, 1, outliers=4, lognormal_scale=False, outlier_channels=ch, bf16=False)
    q = queries(rng, 1, 1, 1, bf16=False)
    nb = (T + BLOCK - 1) // BLOCK
    table = np.arange(nb, dtype=np.int32)[None, :]
    return dict(k=k, v=v, q=q, table=table, num_blocks=nb,
                context_lens=np.array([T], dtype=np.int32),
                slots=slots_for(table, 0, np.arange(T)))


def gqa_case(seed: int, T: int, Hq: int, Hkv: int, q_len: int = 1, shuffle: bool = True):
    """One sequence of T cached tokens (bf16 outlier-channel KV), q_len
    queries; random block table."""
    rng = np.random.default_rng(seed)
    k = kv_tensor(rng, T, Hkv)
    v = kv_tensor(rng, T, Hkv)
    q = queries(rng, 1, q_len, Hq)
    table, nb = block_tables(rng, [T], shuffle=shuffle)
    return dict(k=k, v=v, q=q, table=table, num_blocks=nb,
                context_lens=np.array([T], dtype=np.int32),
                slots=slots_for(table, 0, np.arange(T)))


def ragged_case(seed: int, B: int, Hq: int, Hkv: int, lo: int = 512, hi: int = 32768,
                steps: int = 1, lengths=None):
    """Continuous batching: B sequences with ragged cached lengths, room for
    ``steps`` appended tokens each.  Returns the cached KV per sequence (one
    concatenated batch with its slot mapping) and per-step new tokens."""
    rng = np.random.default_rng(seed)
    L = ragged_lengths(rng, B, lo, hi) if lengths is None else np.asarray(lengths, np.int64)
    table, nb = block_tables(rng, L + steps)
    total = int(L.sum())
    k = kv_tensor(rng, total, Hkv)
    v = kv_tensor(rng, total, Hkv)
    slots = np.concatenate([slots_for(table, b, np.arange(L[b])) for b in range(B)]) \
        if total else np.zeros(0, np.int64)
    new_k = kv_tensor(rng, B * steps, Hkv).reshape(steps, B, Hkv, HEAD_DIM)
    new_v = kv_tensor(rng, B * steps, Hkv).reshape(steps, B, Hkv, HEAD_DIM)
    q = queries(rng, steps * B, 1, Hq).reshape(steps, B, 1, Hq, HEAD_DIM)
    new_slots = np.stack([np.array([slots_for(table, b, [L[b] + s])[0] for b in range(B)])
                          for s in range(steps)])
    return dict(lengths=L, table=table, num_blocks=nb, k=k, v=v, slots=slots,
                new_k=new_k, new_v=new_v, q=q, new_slots=new_slots)
