"""Benchmark of the TurboQuant compressed-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--samples N] [--no-cpu-baseline]

Headline workload: a continuous-batching decode step.  16 sequences with
ragged cached contexts (log-uniform in [512, 32768], seed 3), paged
compressed KV in 16-token blocks behind a random block table, GQA 32 query
heads over 8 KV heads, head_dim 128, bf16 outlier-channel Gaussian KV.  One
step is the whole hot path for that batch: append one new token per sequence
(encode 16 x 8 keys and values into their slots: norm, rotation, 3-bit codes,
residual, QJL signs, paged store), then one decode query per head over each
sequence's whole compressed cache (split-K attention, merge with one inverse
rotation).

Inputs are resident in HBM before timing.  The 256 MB Infinity Cache is
defeated by rotating over enough replicas of the pools that consecutive steps
share no data (> 512 MB in total); every replica grows by one token per
sequence each time it is used.

``value`` is the step's algorithmic bytes (compressed KV read once, block
table, queries, outputs, the appended tokens' inputs and records) divided by
the time of K steps run back to back, in GB/s.  Beside it, from >= 50 steps
that carry HIP events around the encode and the attention call: the median
step, encode and attention times, the attention rate and the roofline of the
attention call (its split and merge kernels; rocprofv3 summaries of both are
under profiles/).

Also reported, each on its own memory before the headline loop:
  * attention_long: decode attention alone at 131,072 tokens, 32 query / 4
    KV heads (split-K across the sequence);
  * prefill: 2,048 new tokens appended to a 32,768-token compressed cache
    (32q/8kv): encode 16,384 + 16,384 vectors, then causal attention of the
    2,048 queries on the matrix cores;
  * encode: one 8,192-token GQA layer (65,536 keys + 65,536 values) with its
    own roofline, and the same layer's decode attention;
  * quality: compressed attention against exact attention on the
    uncompressed K/V of that layer (relative L2 and cosine), reported only;
  * cpu_baseline: the CPU oracle on a bounded sample of the headline step
    (single-thread and all cores, CPU model stated).

Byte counters: ``--counters`` runs only the launches the counter passes
profile (headline attention calls and encodes on cold replicas, then a 512 MiB
copy); ``--traffic-from FETCH_CSV WRITE_CSV`` turns two ``rocprofv3 --pmc``
runs of it into profiles/traffic.json (scaled by the copy's known traffic).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
D = 128
K_REC, V_REC = 68, 50               # compressed bytes per token and KV head
K_PAGE, V_PAGE = 1088, 800

# headline: continuous batching
B3, HQ3, HKV3, SEED3 = 16, 32, 8, 3
METRIC = "compressed-KV decode attention effective HBM GB/s (% peak); encode vectors/s"


# the sources each counted launch is built from (its counters go stale when one changes)
TRAFFIC_SOURCES = {
    "encode_kernel": ("tq_encode.hip", "tq_append.hpp", "tq_common.hpp", "tq_internal.h", "tq_host.cpp"),
    "decode_step_call": ("tq_decode.hip", "tq_append.hpp", "tq_common.hpp", "tq_mfma.hpp", "tq_internal.h",
                         "tq_host.cpp"),
}


def kernel_source_hash(key):
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[key]:
        with open(os.path.join(ROOT, "decode_attention_tq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current sources; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get(key)
    if not k or k.get("source_hash") != kernel_source_hash(key):
        return None
    return k.get("hbm_bytes_per_launch")


def replicas_for(bytes_per_replica: int) -> int:
    return max(2, -(-2 * MALL_BYTES // max(1, bytes_per_replica)) + 1)


def decode_bytes(lengths, hq, hkv, q_len=1, q_elem=2, out_elem=4):
    """Algorithmic bytes of one attention call: every visible compressed
    record once, the block-table entries covering them, queries, outputs and
    context lengths."""
    lengths = np.asarray(lengths, np.int64)
    kv = int(lengths.sum()) * hkv * (K_REC + V_REC)
    table = int(((lengths + 15) // 16).sum()) * 4
    nseq = len(lengths)
    return kv + table + nseq * q_len * hq * D * (q_elem + out_elem) + nseq * 4


def encode_bytes(n_tokens, hkv, in_elem=2):
    """Algorithmic bytes of encoding n_tokens x hkv keys and values: inputs
    read once, records written once, one slot per token."""
    return n_tokens * hkv * (2 * D * in_elem + K_REC + V_REC) + n_tokens * 8


# ---------------------------------------------------------------------------
# headline: continuous-batching decode step

def batch_setup(tq, cb, dev, total_steps, hq=HQ3, hkv=HKV3):
    """Pools (replicas) holding the 16 ragged sequences, the per-step new
    tokens, their slots and context lengths, all resident on the device."""
    import torch
    import synth
    HQ3, HKV3 = hq, hkv  # the step's head counts (locals shadowing the defaults)
    rng = np.random.default_rng(SEED3)
    L = synth.ragged_lengths(rng, B3)
    per_replica = int(L.sum()) * HKV3 * (K_PAGE + V_PAGE) // 16
    R = replicas_for(per_replica)
    appends = -(-total_steps // R) + 1
    table_np, nb = synth.block_tables(rng, L + appends)
    table = torch.from_numpy(table_np).to(dev)
    slots_np = np.concatenate([synth.slots_for(table_np, b, np.arange(L[b])) for b in range(B3)])
    slots = torch.from_numpy(slots_np).to(dev)
    k = synth.kv_tensor_device(31, int(L.sum()), HKV3, dev)
    v = synth.kv_tensor_device(32, int(L.sum()), HKV3, dev)
    pools = []
    for _ in range(R):
        kp = torch.empty((nb, HKV3, K_PAGE), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, HKV3, V_PAGE), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, slots, kp, vp)
        pools.append((kp, vp))
    del k, v
    # step i uses replica i % R and appends token L_b + i // R of every sequence
    nk = synth.kv_tensor_device(33, total_steps * B3, HKV3, dev).reshape(total_steps, B3, HKV3, D)
    nv = synth.kv_tensor_device(34, total_steps * B3, HKV3, dev).reshape(total_steps, B3, HKV3, D)
    a = np.arange(total_steps) // R
    pos = L[None, :] + a[:, None]
    new_slots = np.stack([np.array([synth.slots_for(table_np, b, [pos[i, b]])[0] for b in range(B3)])
                          for i in range(total_steps)])
    new_slots = torch.from_numpy(new_slots.astype(np.int64)).to(dev)
    clens_np = (pos + 1).astype(np.int32)
    clens = torch.from_numpy(clens_np).to(dev)
    qs = torch.from_numpy(synth.queries(rng, 4 * B3, 1, HQ3)).to(dev, torch.bfloat16).reshape(4, B3, 1, HQ3, D)
    max_ctx = int(clens_np.max())
    step_bytes = [decode_bytes(clens_np[i], HQ3, HKV3) + encode_bytes(B3, HKV3) for i in range(total_steps)]
    dec_bytes = [decode_bytes(clens_np[i], HQ3, HKV3) for i in range(total_steps)]
    return dict(L=L, R=R, table=table, pools=pools, nk=nk, nv=nv, new_slots=new_slots, clens=clens,
                qs=qs, max_ctx=max_ctx, step_bytes=step_bytes, dec_bytes=dec_bytes, nb=nb,
                table_np=table_np)


def batch_step_bench(tq, cb, dev, stream, steps, warmup, samples, hq=HQ3, hkv=HKV3):
    import torch
    HQ3, HKV3 = hq, hkv  # the step's head counts (locals shadowing the defaults)
    total = warmup + steps + 2 * (warmup + samples)
    st = batch_setup(tq, cb, dev, total, hq, hkv)
    out = torch.empty((B3, 1, HQ3, D), dtype=torch.float32, device=dev)
    # one buffer serves the step calls and the breakdown's attention calls
    ws = torch.empty(max(tq.tq_decode_step_workspace_bytes(cb, B3, HQ3, HKV3, st["max_ctx"]),
                         tq.tq_decode_workspace_bytes(cb, B3, 1, HQ3, HKV3, st["max_ctx"])), dtype=torch.uint8,
                     device=dev)
    R = st["R"]

    def step(i, ev=None):
        # the step call: append + attention (two launches when fused)
        kp, vp = st["pools"][i % R]
        if ev is not None:
            ev[0].record(stream)
        tq.tq_decode_step(cb, st["nk"][i], st["nv"][i], st["new_slots"][i], st["qs"][i % 4], kp, vp,
                          st["table"], st["clens"][i], st["max_ctx"], out=out, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    def two_calls(i, ev):
        # the same step as its two separate calls (the breakdown)
        kp, vp = st["pools"][i % R]
        ev[0].record(stream)
        tq.tq_encode_kv(cb, st["nk"][i], st["nv"][i], st["new_slots"][i], kp, vp, stream=stream)
        ev[1].record(stream)
        tq.tq_decode_attention(cb, st["qs"][i % 4], kp, vp, st["table"], st["clens"][i], st["max_ctx"], HKV3,
                               out=out, workspace=ws, stream=stream)
        ev[2].record(stream)

    # phase A: K step calls back to back (value)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record(stream)
    for i in range(warmup, warmup + steps):
        step(i)
    t1.record(stream)
    enqueue = time.perf_counter() - w0
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_s = t0.elapsed_time(t1) / 1e3
    s_per_step = max(wall, gpu_s) / steps
    bytes_a = float(np.mean(st["step_bytes"][warmup:warmup + steps]))

    # phase B: sampled step calls with events around each
    base = warmup + steps
    for i in range(base, base + warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(samples)]
    for j in range(samples):
        step(base + warmup + j, evs[j])
    torch.cuda.synchronize()
    step_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    idx = range(base + warmup, base + warmup + samples)
    step_b = float(np.mean([st["step_bytes"][i] for i in idx]))
    # phase C: the same steps as the two separate calls, events between them
    base += warmup + samples
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(samples)]
    for i in range(base, base + warmup):
        two_calls(i, evc[0])
    torch.cuda.synchronize()
    for j in range(samples):
        two_calls(base + warmup + j, evc[j])
    torch.cuda.synchronize()
    enc_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evc]
    dec_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evc]
    idc = range(base + warmup, base + warmup + samples)
    dec_b = float(np.mean([st["dec_bytes"][i] for i in idc]))
    res = dict(
        s_per_step=s_per_step, bytes_per_step=bytes_a, gpu_s=gpu_s, wall_s=wall, enqueue_s=enqueue, replicas=R,
        lengths=[int(x) for x in st["L"]], max_ctx=st["max_ctx"],
        median_step_us=statistics.median(step_us), mean_step_us=float(np.mean(step_us)), sampled_step_bytes=step_b,
        two_calls_median_step_us=statistics.median([a + b for a, b in zip(enc_us, dec_us)]),
        median_encode_us=statistics.median(enc_us), median_attention_us=statistics.median(dec_us),
        mean_attention_us=float(np.mean(dec_us)), attention_bytes=dec_b, samples=samples)
    del st
    return res


def step_gqa32q4kv(tq, cb, dev, stream, steps=100, warmup=10, samples=50):
    """The same continuous-batching step with 32 query heads over 4 KV heads
    (8 per KV head: the step's split pass runs two waves per run of tiles,
    one head tile each)."""
    r = batch_step_bench(tq, cb, dev, stream, steps, warmup, samples, hq=32, hkv=4)
    v = r["bytes_per_step"] / r["s_per_step"] / 1e9
    return {"workload": "continuous-batching decode step as the headline (same lengths and tables), GQA 32q/4kv",
            "q_heads": 32, "kv_heads": 4, "algorithmic_bytes_per_step": round(r["bytes_per_step"]),
            "us_per_step": round(r["s_per_step"] * 1e6, 2), "GBps": round(v, 1),
            "pct_peak": round(100 * v / HBM_PEAK_GBPS, 2), "median_step_us": round(r["median_step_us"], 2),
            "two_calls_median_step_us": round(r["two_calls_median_step_us"], 2)}


# ---------------------------------------------------------------------------
# attention alone over a long context (131,072 tokens, 32q/4kv)

T_LONG, HKV_LONG, HQ = 131072, 4, 32


def long_context_attention(tq, cb, dev, stream, steps=50, warmup=5):
    import torch
    import synth
    nb = T_LONG // 16
    R = replicas_for(nb * HKV_LONG * (K_PAGE + V_PAGE))
    rng = np.random.default_rng(4)
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(41, T_LONG, HKV_LONG, dev)
    v = synth.kv_tensor_device(42, T_LONG, HKV_LONG, dev)
    pools = []
    for _ in range(R):
        kp = torch.empty((nb, HKV_LONG, K_PAGE), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, HKV_LONG, V_PAGE), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, slots, kp, vp, stream=stream)
        pools.append((kp, vp))
    del k, v
    q = torch.from_numpy(synth.queries(rng, 1, 1, HQ)).to(dev, torch.bfloat16)
    clens = torch.tensor([T_LONG], dtype=torch.int32, device=dev)
    out = torch.empty((1, 1, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_workspace_bytes(cb, 1, 1, HQ, HKV_LONG, T_LONG), dtype=torch.uint8,
                     device=dev)
    for i in range(warmup):
        kp, vp = pools[i % R]
        tq.tq_decode_attention(cb, q, kp, vp, table, clens, T_LONG, HKV_LONG, out=out, workspace=ws,
                               stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        kp, vp = pools[(warmup + i) % R]
        tq.tq_decode_attention(cb, q, kp, vp, table, clens, T_LONG, HKV_LONG, out=out, workspace=ws,
                               stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    by = decode_bytes([T_LONG], HQ, HKV_LONG)
    del pools
    return {"workload": "decode attention alone, batch 1, context 131072, GQA 32q/4kv, d128, split-K",
            "context": T_LONG, "q_heads": HQ, "kv_heads": HKV_LONG, "replicas": R, "calls": steps,
            "algorithmic_bytes": by, "us": round(us, 2), "GBps": round(by / (us / 1e6) / 1e9, 1),
            "pct_peak": round(100 * by / (us / 1e6) / 1e9 / HBM_PEAK_GBPS, 2)}


# ---------------------------------------------------------------------------
# chunked prefill: 2,048 new tokens on a 32,768-token compressed cache

def prefill_flops(cached, new, hq):
    """QK^T and PV multiply-adds of causal attention, 2 FLOP each, d = 128:
    query t of the new block sees cached + t + 1 keys."""
    pairs = new * cached + new * (new + 1) // 2
    return 2 * 2 * D * pairs * hq


def prefill_bench(tq, cb, dev, stream, reps=10, warmup=2, cached=32768, new=2048, hkv=8):
    import torch
    import synth
    T = cached + new
    nb = T // 16
    rng = np.random.default_rng(5)
    table_np = rng.permutation(nb).astype(np.int32)[None, :]
    table = torch.from_numpy(table_np).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(51, T, hkv, dev)
    v = synth.kv_tensor_device(52, T, hkv, dev)
    kp = torch.empty((nb, hkv, K_PAGE), dtype=torch.uint8, device=dev)
    vp = torch.empty((nb, hkv, V_PAGE), dtype=torch.uint8, device=dev)
    tq.tq_encode_kv(cb, k[:cached], v[:cached], slots[:cached], kp, vp, stream=stream)
    kn, vn, sn = k[cached:].contiguous(), v[cached:].contiguous(), slots[cached:].contiguous()
    del k, v
    q = torch.from_numpy(synth.queries(rng, 1, new, HQ)).to(dev, torch.bfloat16)
    clens = torch.tensor([T], dtype=torch.int32, device=dev)
    out = torch.empty((1, new, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_workspace_bytes(cb, 1, new, HQ, hkv, T), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        tq.tq_encode_kv(cb, kn, vn, sn, kp, vp, stream=stream)
        tq.tq_decode_attention(cb, q, kp, vp, table, clens, T, hkv, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in evs:
        e[0].record(stream)
        tq.tq_encode_kv(cb, kn, vn, sn, kp, vp, stream=stream)
        e[1].record(stream)
        tq.tq_decode_attention(cb, q, kp, vp, table, clens, T, hkv, out=out, workspace=ws, stream=stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    enc_us = statistics.median([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    att_us = statistics.median([e[1].elapsed_time(e[2]) * 1e3 for e in evs])
    fl = prefill_flops(cached, new, HQ)
    return {"workload": "chunked prefill: 2048 new tokens on a 32768-token compressed cache, GQA 32q/8kv, "
                        "bf16; encode 16384 K + 16384 V, then causal attention on f16 matrix cores",
            "cached": cached, "new": new, "q_heads": HQ, "kv_heads": hkv, "calls": reps,
            "encode_us": round(enc_us, 1), "encode_vectors_per_s": round(2 * new * hkv / (enc_us / 1e6), 1),
            "attention_us": round(att_us, 1), "attention_flop": fl,
            "attention_TFLOPs": round(fl / (att_us / 1e6) / 1e12, 1),
            "attention_pct_f16_mfma_peak": round(100 * fl / (att_us / 1e6) / 1e12 / F16_MFMA_PEAK_TFLOPS, 2),
            "step_us": round(enc_us + att_us, 1)}


# ---------------------------------------------------------------------------
# one 8,192-token layer: encode roofline, its decode, and compression quality

T2, HKV2 = 8192, 8


def layer_bench(tq, cb, dev, stream, samples=50, warmup=5):
    import torch
    import synth
    case = synth.gqa_case(seed=2, T=T2, Hq=HQ, Hkv=HKV2)
    R = replicas_for(2 * T2 * HKV2 * D * 2 + case["num_blocks"] * HKV2 * (K_PAGE + V_PAGE))
    k0 = torch.from_numpy(case["k"]).to(dev, torch.bfloat16)
    v0 = torch.from_numpy(case["v"]).to(dev, torch.bfloat16)
    reps = [dict(k=k0.clone(), v=v0.clone(),
                 kp=torch.zeros((case["num_blocks"], HKV2, K_PAGE), dtype=torch.uint8, device=dev),
                 vp=torch.zeros((case["num_blocks"], HKV2, V_PAGE), dtype=torch.uint8, device=dev))
            for _ in range(R)]
    slots = torch.from_numpy(case["slots"]).to(dev)
    q = torch.from_numpy(case["q"]).to(dev, torch.bfloat16)
    table = torch.from_numpy(case["table"]).to(dev)
    clens = torch.from_numpy(case["context_lens"]).to(dev)
    out = torch.empty((1, 1, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_workspace_bytes(cb, 1, 1, HQ, HKV2, T2), dtype=torch.uint8, device=dev)

    def run(i, ev=None):
        r = reps[i % R]
        if ev:
            ev[0].record(stream)
        tq.tq_encode_kv(cb, r["k"], r["v"], slots, r["kp"], r["vp"], stream=stream)
        if ev:
            ev[1].record(stream)
        tq.tq_decode_attention(cb, q, r["kp"], r["vp"], table, clens, T2, HKV2, out=out, workspace=ws,
                               stream=stream)
        if ev:
            ev[2].record(stream)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(samples)]
    for j in range(samples):
        run(warmup + j, evs[j])
    torch.cuda.synchronize()
    enc = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    dec = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    eb = encode_bytes(T2, HKV2)
    db = decode_bytes([T2], HQ, HKV2)
    enc_mean = float(np.mean(enc))
    ach = eb / (enc_mean / 1e6) / 1e9
    o = out.double().cpu().numpy()[0, 0]

    # quality: the same layer's exact attention on its uncompressed K/V
    scale = 1.0 / math.sqrt(D)
    rl2, cos = [], []
    for hq in range(HQ):
        h = hq // (HQ // HKV2)
        kk = case["k"][:, h].astype(np.float64)
        vv = case["v"][:, h].astype(np.float64)
        s = scale * (kk @ case["q"][0, 0, hq].astype(np.float64))
        w = np.exp(s - s.max())
        exact = (w / w.sum()) @ vv
        rl2.append(np.linalg.norm(o[hq] - exact) / np.linalg.norm(exact))
        cos.append(float(o[hq] @ exact / (np.linalg.norm(o[hq]) * np.linalg.norm(exact))))
    del reps
    # a control with plain N(0, 1) keys and values (4 outlier channels x20,
    # fp32, one head of 1024 tokens): attention there is far less peaked
    c1 = synth.single_head_case(seed=1, T=1024)
    kp1 = torch.zeros((c1["num_blocks"], 1, K_PAGE), dtype=torch.uint8, device=dev)
    vp1 = torch.zeros((c1["num_blocks"], 1, V_PAGE), dtype=torch.uint8, device=dev)
    tq.tq_encode_kv(cb, torch.from_numpy(c1["k"]).to(dev), torch.from_numpy(c1["v"]).to(dev),
                    torch.from_numpy(c1["slots"]).to(dev), kp1, vp1, stream=stream)
    o1 = tq.tq_decode_attention(cb, torch.from_numpy(c1["q"]).to(dev), kp1, vp1,
                                torch.from_numpy(c1["table"]).to(dev),
                                torch.from_numpy(c1["context_lens"]).to(dev), 1024, 1,
                                stream=stream).double().cpu().numpy()[0, 0, 0]
    kk1, vv1 = c1["k"][:, 0].astype(np.float64), c1["v"][:, 0].astype(np.float64)
    s1 = scale * (kk1 @ c1["q"][0, 0, 0].astype(np.float64))
    w1 = np.exp(s1 - s1.max())
    ex1 = (w1 / w1.sum()) @ vv1
    rl2_1 = float(np.linalg.norm(o1 - ex1) / np.linalg.norm(ex1))
    cos_1 = float(o1 @ ex1 / (np.linalg.norm(o1) * np.linalg.norm(ex1)))
    return {
        "encode": {"workload": "one GQA layer: 8192 tokens x 8 KV heads, bf16 outlier-channel KV "
                               "(65536 keys + 65536 values)",
                   "vectors_per_s": round(2 * T2 * HKV2 / (enc_mean / 1e6), 1),
                   "key_vectors_per_s": round(T2 * HKV2 / (enc_mean / 1e6), 1),
                   "mean_us": round(enc_mean, 2), "median_us": round(statistics.median(enc), 2),
                   "samples": samples, "replicas": R,
                   "roofline": {"kernel": "encode_kernel", "bound": "hbm", "achieved": round(ach, 1),
                                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                                "traffic": load_traffic("encode_kernel"), "algorithmic_bytes": eb}},
        "attention": {"workload": "decode attention, batch 1, context 8192, GQA 32q/8kv",
                      "median_us": round(statistics.median(dec), 2),
                      "GBps": round(db / (statistics.median(dec) / 1e6) / 1e9, 1),
                      "algorithmic_bytes": db},
        "quality": {"what": "compressed-cache attention (GPU) against exact float64 softmax attention on the "
                            "uncompressed bf16 K/V of the same layer, 32 query heads; reported, not gated",
                    "rel_l2_mean": round(float(np.mean(rl2)), 5), "rel_l2_max": round(float(np.max(rl2)), 5),
                    "cosine_mean": round(float(np.mean(cos)), 6), "cosine_min": round(float(np.min(cos)), 6),
                    "control_single_head_n01": {"rel_l2": round(rl2_1, 5), "cosine": round(cos_1, 6),
                                                "workload": "1 head, 1024 tokens, fp32 N(0,1) K/V with 4 outlier "
                                                            "channels x20"}},
    }


# ---------------------------------------------------------------------------
# CPU oracle on a bounded sample of the headline step

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(target_s=8.0):
    """The oracle (float64 NumPy, untuned) on sequences of the headline batch,
    taken in order until about target_s of single-thread work: their caches
    encoded (untimed) into pages, then timed: the step's append (one new key
    and value per KV head, encoded and stored) and decode attention of the 32
    query heads over the whole cache.  Run single-threaded, then with all
    BLAS threads.  The rate is the sample's algorithmic bytes per second."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import codebook_fp32, decode_paged, encode_k, encode_v, gaussian_matrix
    from oracle.pages import K_PAGE_BYTES, V_PAGE_BYTES, write_slots_fast
    import synth
    c32, t32 = codebook_fp32(128, 3)
    S = gaussian_matrix(synth.QJL_SEED)
    rng = np.random.default_rng(SEED3)
    L = synth.ragged_lengths(rng, B3)
    data = np.random.default_rng(300)

    def prepare(b):
        n = int(L[b]) + 1
        k = synth.kv_tensor(data, n, HKV3)
        v = synth.kv_tensor(data, n, HKV3)
        table, nb = synth.block_tables(data, [n])
        kp = np.zeros((nb, HKV3, K_PAGE_BYTES), np.uint8)
        vp = np.zeros((nb, HKV3, V_PAGE_BYTES), np.uint8)
        slots = synth.slots_for(table, 0, np.arange(n - 1))
        write_slots_fast(kp, vp, slots, encode_k(k[:-1], c32, t32, S), encode_v(v[:-1], c32, t32))
        q = synth.queries(data, 1, 1, HQ3).astype(np.float64)
        return dict(k=k, v=v, table=table, kp=kp, vp=vp, q=q, n=n,
                    last=synth.slots_for(table, 0, [n - 1]))

    def run(p):
        ek = encode_k(p["k"][-1:], c32, t32, S)
        ev = encode_v(p["v"][-1:], c32, t32)
        write_slots_fast(p["kp"], p["vp"], p["last"], ek, ev)
        decode_paged(p["q"], p["kp"], p["vp"], p["table"], np.array([p["n"]]), c32, S)

    sample, t_single, by = [], 0.0, 0
    for b in range(B3):
        p = prepare(b)  # untimed, all threads
        with threadpool_limits(1):
            t0 = time.perf_counter()
            run(p)
            t_single += time.perf_counter() - t0
        sample.append(p)
        by += decode_bytes([p["n"]], HQ3, HKV3) + encode_bytes(1, HKV3)
        if t_single >= target_s:
            break
    # the whole batch is quicker than the target: repeat it
    reps = max(1, int(math.ceil(target_s / max(t_single, 1e-3)))) if t_single < target_s else 1
    with threadpool_limits(1):
        if reps > 1:
            t0 = time.perf_counter()
            for _ in range(reps):
                for p in sample:
                    run(p)
            t_single = (time.perf_counter() - t0) / reps
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    t0 = time.perf_counter()
    for _ in range(reps):
        for p in sample:
            run(p)
    t_all = (time.perf_counter() - t0) / reps
    lens = [p["n"] for p in sample]
    return {"value": round(by / t_all / 1e9, 5), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "single_thread_value": round(by / t_single / 1e9, 5),
            "sample": (f"{len(sample)} of the 16 sequences of the headline step (contexts {lens}): append one "
                       f"token (encode + store 8 keys and 8 values) and decode attention of 32 query heads over "
                       f"the whole compressed cache, float64 NumPy; {by} algorithmic bytes per pass, "
                       f"{reps} pass(es); {t_single:.2f} s per pass on 1 thread, {t_all:.2f} s on {threads} "
                       f"BLAS threads"),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


# ---------------------------------------------------------------------------
# byte counters

def counters_driver(tq, cb, dev, stream, launches=8):
    """Launches for the rocprofv3 --pmc passes: headline attention calls and
    layer encodes on cold replicas, then 512 MiB device copies (the byte
    counters' calibration)."""
    import torch
    import synth
    st = batch_setup(tq, cb, dev, launches)
    out = torch.empty((B3, 1, HQ3, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_step_workspace_bytes(cb, B3, HQ3, HKV3, st["max_ctx"]), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    for i in range(launches):
        kp, vp = st["pools"][i % st["R"]]
        tq.tq_decode_step(cb, st["nk"][i], st["nv"][i], st["new_slots"][i], st["qs"][0], kp, vp, st["table"],
                          st["clens"][i], st["max_ctx"], out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    del st
    case = synth.gqa_case(seed=2, T=T2, Hq=HQ, Hkv=HKV2)
    k = torch.from_numpy(case["k"]).to(dev, torch.bfloat16)
    v = torch.from_numpy(case["v"]).to(dev, torch.bfloat16)
    slots = torch.from_numpy(case["slots"]).to(dev)
    R = replicas_for(2 * T2 * HKV2 * D * 2)
    reps = [(k.clone(), v.clone(), torch.zeros((case["num_blocks"], HKV2, K_PAGE), dtype=torch.uint8, device=dev),
             torch.zeros((case["num_blocks"], HKV2, V_PAGE), dtype=torch.uint8, device=dev)) for _ in range(R)]
    torch.cuda.synchronize()
    for i in range(launches):
        kk, vv, kp, vp = reps[i % R]
        tq.tq_encode_kv(cb, kk, vv, slots, kp, vp, stream=stream)
    torch.cuda.synchronize()
    a = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def traffic_from(fetch_csv, write_csv):
    """profiles/traffic.json from two counter runs of --counters: per launch
    of each kernel, FETCH_SIZE and WRITE_SIZE scaled by what the same counters
    read for the 512 MiB copy (its true traffic: 512 MiB read, 512 MiB
    written).  The headline decode step call is its prep, split and merge
    kernels."""
    import csv

    def load(path, counter):
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        by = {}
        for (_, name), val in per.items():
            by.setdefault(name, []).append(val)
        return by
    f, w = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")

    def calib(by):
        cp = [v for n, vals in by.items() if "copy" in n.lower() for v in vals]
        big = max(cp)
        cp = sorted(v for v in cp if v >= 0.5 * big)
        return (512 << 20) / cp[len(cp) // 2]
    fs, wsc = calib(f), calib(w)

    def med(by, needle, scale):
        vals = sorted(v for n, vs in by.items() if needle in n for v in vs)
        return vals[len(vals) // 2] * scale if vals else None
    rec = {}
    enc_f, enc_w = med(f, "encode_kernel", fs), med(w, "encode_kernel", wsc)
    rec["encode_kernel"] = {"source_hash": kernel_source_hash("encode_kernel"), "workload": "one 8192-token layer, 8 KV heads",
                            "hbm_bytes_per_launch": round(enc_f + enc_w), "fetch_bytes": round(enc_f),
                            "write_bytes": round(enc_w), "algorithmic_bytes": encode_bytes(T2, HKV2)}
    parts = {}
    for needle in ("step_prep_kernel", "split_", "merge_kernel"):
        ff, ww = med(f, needle, fs), med(w, needle, wsc)
        if ff is not None:
            parts[needle.strip("_")] = {"fetch_bytes": round(ff), "write_bytes": round(ww)}
    import synth
    L = synth.ragged_lengths(np.random.default_rng(SEED3), B3)
    tot = sum(p["fetch_bytes"] + p["write_bytes"] for p in parts.values())
    rec["decode_step_call"] = {"source_hash": kernel_source_hash("decode_step_call"), "workload": "decode step of 16 ragged sequences, 32q/8kv",
                               "hbm_bytes_per_launch": round(tot), "kernels": parts,
                               "algorithmic_bytes_at_cached_lengths": decode_bytes(L + 1, HQ3, HKV3)
                               + encode_bytes(B3, HKV3)}
    rec["copy_calibration"] = {"fetch_bytes_per_counter_unit": fs, "write_bytes_per_counter_unit": wsc}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps(rec))


# ---------------------------------------------------------------------------

def hot_window_attention(tq, cb, dev, stream, steps=30, warmup=5, T=8192, W=2048):
    """Decode with an exact bf16 hot window of W recent tokens after T
    compressed ones (32q/8kv), the window at the pages' 2,048-token threshold."""
    import torch
    import synth
    hkv = 8
    nb = T // 16
    R = replicas_for(nb * hkv * (K_PAGE + V_PAGE) + W * hkv * D * 2 * 2)
    rng = np.random.default_rng(5)
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(41, T, hkv, dev)
    v = synth.kv_tensor_device(42, T, hkv, dev)
    reps = []
    for r in range(R):
        kp = torch.empty((nb, hkv, K_PAGE), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, hkv, V_PAGE), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, slots, kp, vp, stream=stream)
        hk = synth.kv_tensor_device(100 + 2 * r, W, hkv, dev).reshape(1, W, hkv, D)
        hv = synth.kv_tensor_device(101 + 2 * r, W, hkv, dev).reshape(1, W, hkv, D)
        reps.append((kp, vp, hk, hv))
    del k, v
    q = torch.from_numpy(synth.queries(rng, 1, 1, HQ)).to(dev, torch.bfloat16)
    clens = torch.tensor([T], dtype=torch.int32, device=dev)
    hlens = torch.tensor([W], dtype=torch.int32, device=dev)
    out = torch.empty((1, 1, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_hot_workspace_bytes(cb, 1, HQ, hkv, T, W), dtype=torch.uint8, device=dev)

    def call(i):
        kp, vp, hk, hv = reps[i % R]
        tq.tq_decode_attention_hot(cb, q, kp, vp, table, clens, T, hkv, hk, hv, hlens, out=out,
                                   workspace=ws, stream=stream)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        call(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    by = decode_bytes([T], HQ, hkv) + W * hkv * D * 2 * 2 + 4
    del reps
    return {"context": T, "hot_window": W, "q_heads": HQ, "kv_heads": hkv, "replicas": R,
            "algorithmic_bytes": by, "us": round(us, 2), "GBps": round(by / (us / 1e6) / 1e9, 1),
            "pct_peak": round(100 * by / (us / 1e6) / 1e9 / HBM_PEAK_GBPS, 2)}


def verify_attention(tq, cb, dev, stream, steps=30, warmup=5, T=32768, q_lens=(1, 2, 4, 8)):
    """Multi-token verify decode: q_len new tokens per sequence (causal over
    the block) over T compressed tokens, 32q/8kv."""
    import torch
    import synth
    hkv = 8
    nb = T // 16
    R = replicas_for(nb * hkv * (K_PAGE + V_PAGE))
    rng = np.random.default_rng(6)
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(41, T, hkv, dev)
    v = synth.kv_tensor_device(42, T, hkv, dev)
    pools = []
    for _ in range(R):
        kp = torch.empty((nb, hkv, K_PAGE), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, hkv, V_PAGE), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, slots, kp, vp, stream=stream)
        pools.append((kp, vp))
    del k, v
    clens = torch.tensor([T], dtype=torch.int32, device=dev)
    res = {"context": T, "q_heads": HQ, "kv_heads": hkv, "replicas": R, "us_per_call": {}}
    for q_len in q_lens:
        q = torch.from_numpy(synth.queries(rng, 1, q_len, HQ)).to(dev, torch.bfloat16)
        out = torch.empty((1, q_len, HQ, D), dtype=torch.float32, device=dev)
        ws = torch.empty(tq.tq_decode_workspace_bytes(cb, 1, q_len, HQ, hkv, T), dtype=torch.uint8, device=dev)
        for i in range(warmup):
            kp, vp = pools[i % R]
            tq.tq_decode_attention(cb, q, kp, vp, table, clens, T, hkv, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            kp, vp = pools[(warmup + i) % R]
            tq.tq_decode_attention(cb, q, kp, vp, table, clens, T, hkv, out=out, workspace=ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res["us_per_call"][str(q_len)] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    del pools
    return res


def window_attention(tq, cb, dev, stream, steps=30, warmup=5, W=1024):
    """Sliding-window decode over a rotating cache: the headline batch's 16
    ragged sequences (contexts log-uniform in [512, 32768]), 32q/8kv, a
    1,024-token window (the pages' Gemma 4 sliding layers) over a ring of
    65 pages per sequence; only the pages the window overlaps are read."""
    import torch
    import synth
    hkv, R_ring = 8, 65
    rng = np.random.default_rng(SEED3)
    L = synth.ragged_lengths(rng, B3)
    per_rep = B3 * R_ring * hkv * (K_PAGE + V_PAGE)
    R = replicas_for(per_rep)
    nb = B3 * R_ring
    table_np = rng.permutation(nb).astype(np.int32).reshape(B3, R_ring)
    table = torch.from_numpy(table_np).to(dev)
    # the last 16 R_ring positions of every sequence, written once (older ones
    # would be overwritten by them)
    pos = [np.arange(max(0, int(l) - 16 * R_ring), int(l)) for l in L]
    slots = np.concatenate([table_np[b][(p // 16) % R_ring].astype(np.int64) * 16 + p % 16
                            for b, p in enumerate(pos)])
    n = len(slots)
    k = synth.kv_tensor_device(61, n, hkv, dev)
    v = synth.kv_tensor_device(62, n, hkv, dev)
    st = torch.from_numpy(slots).to(dev)
    pools = []
    for _ in range(R):
        kp = torch.empty((nb, hkv, K_PAGE), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, hkv, V_PAGE), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, st, kp, vp, stream=stream)
        pools.append((kp, vp))
    del k, v
    q = torch.from_numpy(synth.queries(rng, B3, 1, HQ)).to(dev, torch.bfloat16)
    clens = torch.from_numpy(L.astype(np.int32)).to(dev)
    out = torch.empty((B3, 1, HQ, D), dtype=torch.float32, device=dev)
    maxc = int(L.max())
    ws = torch.empty(tq.tq_decode_window_workspace_bytes(cb, B3, 1, HQ, hkv, maxc, W), dtype=torch.uint8, device=dev)

    def call(i):
        kp, vp = pools[i % R]
        tq.tq_decode_attention_window(cb, q, kp, vp, table, clens, maxc, hkv, W, out=out, workspace=ws,
                                      stream=stream)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        call(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    by = decode_bytes(np.minimum(L, W), HQ, hkv)
    del pools
    return {"workload": "sliding-window decode, batch 16 ragged contexts (headline lengths), window 1024, "
                        "ring of 65 pages per sequence, GQA 32q/8kv",
            "window": W, "ring_pages": R_ring, "replicas": R, "calls": steps, "algorithmic_bytes": by,
            "us": round(us, 2), "GBps": round(by / (us / 1e6) / 1e9, 1),
            "pct_peak": round(100 * by / (us / 1e6) / 1e9 / HBM_PEAK_GBPS, 2)}


def bits_variants(tq, dev, stream, steps=20, warmup=3):
    """The 2- and 4-bit codebook variants on one 8,192-token GQA layer
    (32q/8kv): encode of the layer and its decode attention (vector pass),
    beside the 3-bit pages' method."""
    import torch
    import synth
    case = synth.gqa_case(seed=2, T=T2, Hq=HQ, Hkv=HKV2)
    k = torch.from_numpy(case["k"]).to(dev, torch.bfloat16)
    v = torch.from_numpy(case["v"]).to(dev, torch.bfloat16)
    slots = torch.from_numpy(case["slots"]).to(dev)
    q = torch.from_numpy(case["q"]).to(dev, torch.bfloat16)
    table = torch.from_numpy(case["table"]).to(dev)
    clens = torch.from_numpy(case["context_lens"]).to(dev)
    res = {"workload": "one GQA layer: 8192 tokens x 8 KV heads, bf16; encode, then 1 query per head"}
    for bits in (2, 3, 4):
        cbb = tq.tq_codebook_init(128, bits, synth.QJL_SEED, device=dev)
        kb, vb = tq.tq_k_page_bytes(cbb), tq.tq_v_page_bytes(cbb)
        kp = torch.zeros((case["num_blocks"], HKV2, kb), dtype=torch.uint8, device=dev)
        vp = torch.zeros((case["num_blocks"], HKV2, vb), dtype=torch.uint8, device=dev)
        out = torch.empty((1, 1, HQ, D), dtype=torch.float32, device=dev)
        ws = torch.empty(tq.tq_decode_workspace_bytes(cbb, 1, 1, HQ, HKV2, T2), dtype=torch.uint8, device=dev)
        for _ in range(warmup):
            tq.tq_encode_kv(cbb, k, v, slots, kp, vp, stream=stream)
            tq.tq_decode_attention(cbb, q, kp, vp, table, clens, T2, HKV2, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in evs:
            e[0].record(stream)
            tq.tq_encode_kv(cbb, k, v, slots, kp, vp, stream=stream)
            e[1].record(stream)
            tq.tq_decode_attention(cbb, q, kp, vp, table, clens, T2, HKV2, out=out, workspace=ws, stream=stream)
            e[2].record(stream)
        torch.cuda.synchronize()
        enc = statistics.median([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
        att = statistics.median([e[1].elapsed_time(e[2]) * 1e3 for e in evs])
        kv_bytes = T2 * HKV2 * (kb + vb) // 16
        res[f"{bits}bit"] = {"k_page_bytes": kb, "v_page_bytes": vb,
                             "bits_per_coordinate": round((kb + vb) * 8 / (2 * 16 * D), 4),
                             "encode_us": round(enc, 2), "attention_us": round(att, 2),
                             "attention_GBps": round((kv_bytes + HQ * D * 6) / (att / 1e6) / 1e9, 1),
                             "decode_pass": "matrix cores" if bits == 3 else "vector"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--samples", type=int, default=60, help="event-timed steps (>= 50)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the continuous-batching step (for kernel traces of it)")
    ap.add_argument("--counters", action="store_true",
                    help="only run the launches that the byte-counter passes profile")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two counter runs of --counters")
    ap.add_argument("--long-context-only", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--verify-only", action="store_true")
    ap.add_argument("--hot-window-only", action="store_true")
    ap.add_argument("--window-only", action="store_true")
    ap.add_argument("--bits-only", action="store_true")
    ap.add_argument("--step-32q4kv-only", action="store_true")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the method's multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_tq_amd as tq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    cb = tq.tq_codebook_init(128, 3, synth.QJL_SEED, device=dev)
    if args.counters:
        counters_driver(tq, cb, dev, stream)
        return
    if args.verify_only:
        print(json.dumps({"attention_verify": verify_attention(tq, cb, dev, stream, steps=args.steps,
                                                               warmup=args.warmup)}))
        return
    if args.hot_window_only:
        print(json.dumps({"attention_hot_window": hot_window_attention(tq, cb, dev, stream, steps=args.steps,
                                                                       warmup=args.warmup)}))
        return
    if args.window_only:
        print(json.dumps({"attention_window": window_attention(tq, cb, dev, stream, steps=args.steps,
                                                               warmup=args.warmup)}))
        return
    if args.bits_only:
        print(json.dumps({"bits_variants": bits_variants(tq, dev, stream, steps=args.steps, warmup=args.warmup)}))
        return
    if args.long_context_only:
        print(json.dumps({"attention_long": long_context_attention(tq, cb, dev, stream, steps=args.steps,
                                                                   warmup=args.warmup)}))
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_bench(tq, cb, dev, stream, reps=args.steps, warmup=args.warmup)}))
        return
    if args.step_32q4kv_only:
        print(json.dumps({"decode_step_gqa32q4kv": step_gqa32q4kv(tq, cb, dev, stream, steps=args.steps,
                                                                  warmup=args.warmup)}))
        return

    extra = {}
    if not args.headline_only:
        sides = (("attention_long", lambda: long_context_attention(tq, cb, dev, stream)),
                 ("prefill", lambda: prefill_bench(tq, cb, dev, stream)),
                 ("layer_8192", lambda: layer_bench(tq, cb, dev, stream)),
                 ("attention_verify", lambda: verify_attention(tq, cb, dev, stream)),
                 ("attention_hot_window", lambda: hot_window_attention(tq, cb, dev, stream)),
                 ("attention_window", lambda: window_attention(tq, cb, dev, stream)),
                 ("decode_step_gqa32q4kv", lambda: step_gqa32q4kv(tq, cb, dev, stream)),
                 ("bits_variants", lambda: bits_variants(tq, dev, stream)))
        for key, run in sides:
            extra[key] = run()
            torch.cuda.empty_cache()
            print(json.dumps({"progress": key + " done"}), file=sys.stderr, flush=True)

    res = batch_step_bench(tq, cb, dev, stream, args.steps, args.warmup, max(args.samples, 50))
    value = res["bytes_per_step"] / res["s_per_step"] / 1e9
    step_mean = res["mean_step_us"]
    achieved = res["sampled_step_bytes"] / (step_mean / 1e6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res["s_per_step"] * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "continuous-batching decode step: batch 16, ragged contexts log-uniform in "
                               "[512, 32768] (seed 3), 16-token pages behind a random block table, GQA 32q/8kv, "
                               "d128, bf16 outlier-channel KV; step = append and encode 1 K/V per sequence "
                               "(16 x 8 keys + values) + decode attention of 1 query per head over the whole "
                               "compressed cache",
                   "batch": B3, "q_heads": HQ3, "kv_heads": HKV3, "head_dim": D,
                   "context_lengths": res["lengths"], "replicas": res["replicas"],
                   "algorithmic_bytes_per_step": round(res["bytes_per_step"])},
        "pct_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "median_step_us": round(res["median_step_us"], 2),
        "timed_region": {"wall_s": round(res["wall_s"], 6), "gpu_event_s": round(res["gpu_s"], 6),
                         "host_enqueue_s": round(res["enqueue_s"], 6)},
        "two_calls": {"median_step_us": round(res["two_calls_median_step_us"], 2),
                      "median_encode_us": round(res["median_encode_us"], 2),
                      "median_attention_us": round(res["median_attention_us"], 2),
                      "attention_GBps_median": round(res["attention_bytes"] / (res["median_attention_us"] / 1e6)
                                                     / 1e9, 1)},
        "event_samples": res["samples"],
        "roofline": {"kernel": "decode step call (step_prep_kernel + split_wave_kernel + merge_kernel)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic("decode_step_call"),
                     "avg_launch_us": round(step_mean, 2), "algorithmic_bytes": round(res["sampled_step_bytes"])},
    }
    line.update(extra)
    if extra:
        line["encode_vectors_per_s"] = extra["layer_8192"]["encode"]["vectors_per_s"]
    if not args.no_cpu_baseline and not args.headline_only:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
