"""Benchmark of the TurboQuant compressed-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (default): one GQA decode layer, 32 query heads over 8 KV heads,
head_dim 128, batch 1, 8192 cached tokens of bf16 outlier-channel Gaussian
KV.  One step is the whole hot path: encode the full cache (65,536 key and
65,536 value vectors: norm, rotation, 3-bit codes, residual, QJL signs, paged
store) and one decode query per head over the compressed cache (split-K
attention forming its own query operands, merge with one inverse rotation).

Inputs are resident in HBM before timing.  The 256 MB Infinity Cache is
defeated by rotating over enough independent replicas of inputs and pools
that consecutive steps never share data (> 512 MB in total).

Prints one JSON line: the whole step's effective HBM rate (algorithmic bytes /
time) as ``value``, the encode rate in vectors/s and the attention rate in
GB/s alongside, the decode attention rate on its own over a long context
(131,072 tokens, 32 query / 4 KV heads) as ``attention_long``, the roofline
of the dominant kernel from HIP events recorded around it on its stream, and
the CPU oracle timed on the host for the same step.  A timing event costs the
stream a few microseconds, so inside the timed steps only every tenth step
carries events (around its encode and its attention call); the long-context
rate is measured first, on its own memory.

Byte counters: ``--counters`` runs only encode launches and a 512 MiB copy,
for two ``rocprofv3 --pmc`` passes (FETCH_SIZE, then WRITE_SIZE);
``--traffic-from FETCH_CSV WRITE_CSV`` turns them into profiles/traffic.json
(scaled by the copy's known traffic).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
SAMPLE = 10  # timed steps per step that carries timing events

T, HQ, HKV, D = 8192, 32, 8, 128
WORKLOAD = ("GQA decode layer: 32 q-heads / 8 KV heads, d=128, batch 1, context 8192, "
            "bf16 outlier-channel KV; step = encode full cache (65536 K + 65536 V vectors) "
            "+ 1 decode query per head")


def algorithmic_bytes():
    """Bytes a step must move at minimum (inputs read once, outputs written once)."""
    per_tok = HKV * (2 * D * 2 + 68 + 50) + 8          # bf16 K and V in, records out, slot
    encode = T * per_tok
    blocks = T // 16
    decode = T * HKV * 118 + blocks * 4 + HQ * D * 2 + HQ * D * 4 + 4
    return encode, decode


def encode_flops_per_key():
    # QJL projection 2*m*d plus two rotations, norm, residual (small terms)
    return 2 * 128 * 128 + 2 * 7 * 128 + 6 * 128


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("tq_encode.hip", "tq_decode.hip", "tq_common.hpp", "tq_mfma.hpp", "tq_internal.h"):
        with open(os.path.join(ROOT, "decode_attention_tq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get(kernel)
    if not k or k.get("source_hash") != kernel_source_hash():
        return None
    return k.get("hbm_bytes_per_launch")


# Long-context decode: one query per head over 131,072 compressed tokens,
# 32 query heads over 4 KV heads (the decode attention rate on its own).
T_LONG, HKV_LONG = 131072, 4


def long_context_attention(tq, cb, dev, stream, steps=30, warmup=5):
    """Decode attention alone over a long compressed context: pages encoded
    from device-drawn outlier-channel bf16 KV, rotated over enough replicas
    that consecutive calls share no data through the 256 MB Infinity Cache."""
    import torch
    import synth
    nb = T_LONG // 16
    per_replica = nb * HKV_LONG * (1088 + 800)
    R = max(2, -(-2 * MALL_BYTES // per_replica) + 1)
    rng = np.random.default_rng(4)
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(41, T_LONG, HKV_LONG, dev)
    v = synth.kv_tensor_device(42, T_LONG, HKV_LONG, dev)
    pools = []
    for r in range(R):
        kp = torch.empty((nb, HKV_LONG, 1088), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, HKV_LONG, 800), dtype=torch.uint8, device=dev)
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
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        kp, vp = pools[(warmup + i) % R]
        tq.tq_decode_attention(cb, q, kp, vp, table, clens, T_LONG, HKV_LONG, out=out, workspace=ws,
                               stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    by = T_LONG * HKV_LONG * 118 + nb * 4 + HQ * D * 2 + HQ * D * 4 + 4
    del pools
    return {"context": T_LONG, "q_heads": HQ, "kv_heads": HKV_LONG, "replicas": R,
            "algorithmic_bytes": by, "us": round(us, 2), "GBps": round(by / (us / 1e6) / 1e9, 1),
            "pct_peak": round(100 * by / (us / 1e6) / 1e9 / HBM_PEAK_GBPS, 2)}


def hot_window_attention(tq, cb, dev, stream, steps=30, warmup=5, T=8192, W=2048):
    """Decode with an exact bf16 hot window of W recent tokens after T
    compressed ones (32q/8kv): the deployment the pages describe, with the
    window at their 2,048-token compression threshold.  Replicas rotate so
    that consecutive calls share no data through the Infinity Cache."""
    import torch
    import synth
    nb = T // 16
    per_replica = nb * HKV * (1088 + 800) + W * HKV * D * 2 * 2
    R = max(2, -(-2 * MALL_BYTES // per_replica) + 1)
    rng = np.random.default_rng(5)
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(41, T, HKV, dev)
    v = synth.kv_tensor_device(42, T, HKV, dev)
    reps = []
    for r in range(R):
        kp = torch.empty((nb, HKV, 1088), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, HKV, 800), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, slots, kp, vp, stream=stream)
        hk = synth.kv_tensor_device(100 + 2 * r, W, HKV, dev).to(torch.bfloat16).reshape(1, W, HKV, D)
        hv = synth.kv_tensor_device(101 + 2 * r, W, HKV, dev).to(torch.bfloat16).reshape(1, W, HKV, D)
        reps.append((kp, vp, hk, hv))
    del k, v
    q = torch.from_numpy(synth.queries(rng, 1, 1, HQ)).to(dev, torch.bfloat16)
    clens = torch.tensor([T], dtype=torch.int32, device=dev)
    hlens = torch.tensor([W], dtype=torch.int32, device=dev)
    out = torch.empty((1, 1, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_hot_workspace_bytes(cb, 1, HQ, HKV, T, W), dtype=torch.uint8, device=dev)

    def call(i):
        kp, vp, hk, hv = reps[i % R]
        tq.tq_decode_attention_hot(cb, q, kp, vp, table, clens, T, HKV, hk, hv, hlens, out=out,
                                   workspace=ws, stream=stream)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        call(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    by = T * HKV * 118 + W * HKV * D * 2 * 2 + nb * 4 + HQ * D * 2 + HQ * D * 4 + 8
    del reps
    return {"context": T, "hot_window": W, "q_heads": HQ, "kv_heads": HKV, "replicas": R,
            "algorithmic_bytes": by, "us": round(us, 2), "GBps": round(by / (us / 1e6) / 1e9, 1),
            "pct_peak": round(100 * by / (us / 1e6) / 1e9 / HBM_PEAK_GBPS, 2)}


def verify_attention(tq, cb, dev, stream, steps=30, warmup=5, T=32768, q_lens=(1, 2, 4, 8)):
    """Multi-token verify decode: q_len new tokens per sequence (causal over
    the block) over T compressed tokens, 32q/8kv, the pages' speculative /
    multi-token decoding step.  Replicas rotate beyond the Infinity Cache."""
    import torch
    import synth
    nb = T // 16
    per_replica = nb * HKV * (1088 + 800)
    R = max(2, -(-2 * MALL_BYTES // per_replica) + 1)
    rng = np.random.default_rng(6)
    table = torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev)
    slots = (table[0].to(torch.int64)[:, None] * 16 + torch.arange(16, device=dev)).reshape(-1)
    k = synth.kv_tensor_device(41, T, HKV, dev)
    v = synth.kv_tensor_device(42, T, HKV, dev)
    pools = []
    for r in range(R):
        kp = torch.empty((nb, HKV, 1088), dtype=torch.uint8, device=dev)
        vp = torch.empty((nb, HKV, 800), dtype=torch.uint8, device=dev)
        tq.tq_encode_kv(cb, k, v, slots, kp, vp, stream=stream)
        pools.append((kp, vp))
    del k, v
    clens = torch.tensor([T], dtype=torch.int32, device=dev)
    res = {"context": T, "q_heads": HQ, "kv_heads": HKV, "replicas": R, "us_per_call": {}}
    for q_len in q_lens:
        q = torch.from_numpy(synth.queries(rng, 1, q_len, HQ)).to(dev, torch.bfloat16)
        out = torch.empty((1, q_len, HQ, D), dtype=torch.float32, device=dev)
        ws = torch.empty(tq.tq_decode_workspace_bytes(cb, 1, q_len, HQ, HKV, T), dtype=torch.uint8, device=dev)
        for i in range(warmup):
            kp, vp = pools[i % R]
            tq.tq_decode_attention(cb, q, kp, vp, table, clens, T, HKV, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            kp, vp = pools[(warmup + i) % R]
            tq.tq_decode_attention(cb, q, kp, vp, table, clens, T, HKV, out=out, workspace=ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res["us_per_call"][str(q_len)] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    del pools
    return res


def counters_driver(tq, cb, dev, stream, reps, case_slots, launches=8):
    """Launches for rocprofv3 --pmc passes: encode launches on cold replicas,
    then plain device copies of 512 MiB (calibration of the byte counters)."""
    import torch
    for i in range(launches):
        r = reps[i % len(reps)]
        tq.tq_encode_kv(cb, r["k"], r["v"], case_slots, r["kp"], r["vp"], stream=stream)
    torch.cuda.synchronize()
    a = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def traffic_from(fetch_csv, write_csv):
    """profiles/traffic.json from two counter runs of --counters: per encode
    launch, FETCH_SIZE and WRITE_SIZE scaled by what the same counters read
    for the 512 MiB copy (its true traffic: 512 MiB read, 512 MiB written)."""
    import csv
    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        per = {}
        for r in rows:
            per.setdefault((r["Dispatch_Id"], r["Kernel_Name"]), 0.0)
            per[(r["Dispatch_Id"], r["Kernel_Name"])] += float(r["Counter_Value"])
        enc = [v for (d, n), v in per.items() if "encode_kernel" in n]
        # the 512 MiB calibration copies are the largest copies of the run
        cpy = [v for (d, n), v in per.items() if "copy" in n.lower()]
        big = max(cpy)
        cpy = [v for v in cpy if v >= 0.5 * big]
        return sorted(enc), sorted(cpy)
    ef, cf = load(fetch_csv, "FETCH_SIZE")
    ew, cw = load(write_csv, "WRITE_SIZE")
    true = 512 << 20
    f_scale = true / cf[len(cf) // 2]
    w_scale = true / cw[len(cw) // 2]
    fetch = ef[len(ef) // 2] * f_scale
    write = ew[len(ew) // 2] * w_scale
    enc_b, _ = algorithmic_bytes()
    rec = {"encode_kernel": {"source_hash": kernel_source_hash(), "hbm_bytes_per_launch": round(fetch + write),
                             "fetch_bytes": round(fetch), "write_bytes": round(write),
                             "algorithmic_bytes": enc_b,
                             "copy_calibration": {"fetch_bytes_per_counter_unit": f_scale,
                                                  "write_bytes_per_counter_unit": w_scale}}}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(case, target_s=10.0, max_s=30.0):
    """The oracle (float64 NumPy) on the same step, repeated for ~10 s."""
    from threadpoolctl import threadpool_info
    from oracle import codebook_fp32, decode_paged, encode_k, encode_v, gaussian_matrix
    from oracle.pages import K_PAGE_BYTES, V_PAGE_BYTES, write_slots_fast
    import synth
    c32, t32 = codebook_fp32(128, 3)
    S = gaussian_matrix(synth.QJL_SEED)
    reps = 0
    t0 = time.perf_counter()
    while True:
        ek = encode_k(case["k"], c32, t32, S)
        ev = encode_v(case["v"], c32, t32)
        kp = np.zeros((case["num_blocks"], HKV, K_PAGE_BYTES), np.uint8)
        vp = np.zeros((case["num_blocks"], HKV, V_PAGE_BYTES), np.uint8)
        write_slots_fast(kp, vp, case["slots"], ek, ev)
        decode_paged(case["q"], kp, vp, case["table"], case["context_lens"], c32, S)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el + el / reps > max_s:
            break
    enc_b, dec_b = algorithmic_bytes()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round((enc_b + dec_b) * reps / el / 1e9, 4), "unit": "GB/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"the full step (same workload) run {reps}x in {el:.1f} s, float64 NumPy, "
                      f"{threads} BLAS threads on {os.cpu_count()} host cpus",
            "s_per_step": round(el / reps, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="only run the launches that the byte-counter passes profile")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two counter runs of --counters")
    ap.add_argument("--long-context-only", action="store_true",
                    help="only the long-context decode measurement (for kernel traces of it)")
    ap.add_argument("--verify-only", action="store_true",
                    help="only multi-token verify decode (q_len 1, 2, 4, 8) over 32,768 compressed tokens")
    ap.add_argument("--hot-window-only", action="store_true",
                    help="only the decode with an exact 2,048-token window after 8,192 compressed tokens")
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
    cb = tq.tq_codebook_init(128, 3, synth.QJL_SEED, device=dev)
    if args.verify_only:
        print(json.dumps({"attention_verify": verify_attention(
            tq, cb, dev, torch.cuda.current_stream(dev), steps=args.steps, warmup=args.warmup)}))
        return
    if args.hot_window_only:
        print(json.dumps({"attention_hot_window": hot_window_attention(
            tq, cb, dev, torch.cuda.current_stream(dev), steps=args.steps, warmup=args.warmup)}))
        return
    if args.long_context_only:
        print(json.dumps({"attention_long": long_context_attention(
            tq, cb, dev, torch.cuda.current_stream(dev), steps=args.steps, warmup=args.warmup)}))
        return
    long_res = None
    if not args.no_long_context and not args.counters:
        long_res = long_context_attention(tq, cb, dev, torch.cuda.current_stream(dev))
        torch.cuda.empty_cache()
    case = synth.gqa_case(seed=2, T=T, Hq=HQ, Hkv=HKV)

    enc_b, dec_b = algorithmic_bytes()
    per_replica = 2 * T * HKV * D * 2 + case["num_blocks"] * HKV * (1088 + 800)
    R = max(2, -(-2 * MALL_BYTES // per_replica) + 1)
    k0 = torch.from_numpy(case["k"]).to(dev, torch.bfloat16)
    v0 = torch.from_numpy(case["v"]).to(dev, torch.bfloat16)
    reps = []
    for r in range(R):
        reps.append(dict(
            k=k0.clone(), v=v0.clone(),
            kp=torch.zeros((case["num_blocks"], HKV, 1088), dtype=torch.uint8, device=dev),
            vp=torch.zeros((case["num_blocks"], HKV, 800), dtype=torch.uint8, device=dev)))
    slots = torch.from_numpy(case["slots"]).to(dev)
    q = torch.from_numpy(case["q"]).to(dev, torch.bfloat16)
    table = torch.from_numpy(case["table"]).to(dev)
    clens = torch.from_numpy(case["context_lens"]).to(dev)
    out = torch.empty((1, 1, HQ, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_decode_workspace_bytes(cb, 1, 1, HQ, HKV, T), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.counters:
        counters_driver(tq, cb, dev, stream, reps, slots)
        return

    def step(i, ev=None):
        r = reps[i % R]
        if ev is not None:
            ev[0].record(stream)
        tq.tq_encode_kv(cb, r["k"], r["v"], slots, r["kp"], r["vp"], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        tq.tq_decode_attention(cb, q, r["kp"], r["vp"], table, clens, T, HKV, out=out,
                               workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # events on every SAMPLE-th timed step (each event costs the stream time)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] if i % SAMPLE == 0 else None
           for i in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = t_start.elapsed_time(t_end)
    total_s = max(wall, gpu_ms / 1e3)
    ms_per_step = total_s * 1e3 / args.steps
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs if e is not None]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs if e is not None]))

    value = (enc_b + dec_b) / (ms_per_step / 1e3) / 1e9
    n_vec = 2 * T * HKV
    # dominant kernel: the single-launch encode kernel (the attention call is
    # two launches: the split pass, which forms its own query operands, and the merge)
    if enc_ms >= dec_ms:
        name, dur_ms, traffic = "encode_kernel", enc_ms, load_traffic("encode_kernel")
        achieved = enc_b / (dur_ms / 1e3) / 1e9
        roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "avg_launch_us": round(dur_ms * 1e3, 2),
                # key-path work counted as fp32 FLOPs (QJL projection, rotations);
                # the kernel runs the products on the matrix cores
                "nominal_key_tflops": round(T * HKV * encode_flops_per_key() / (dur_ms / 1e3) / 1e12, 2)}
    else:
        name, dur_ms, traffic = "attention (split+merge)", dec_ms, load_traffic("attention")
        achieved = dec_b / (dur_ms / 1e3) / 1e9
        roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "avg_launch_us": round(dur_ms * 1e3, 2)}

    line = {
        "metric": "compressed-KV decode attention effective HBM GB/s (% peak); encode vectors/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": 1, "context": T, "q_heads": HQ, "kv_heads": HKV,
                   "head_dim": D, "kv_dtype": "bf16", "replicas": R,
                   "algorithmic_bytes_per_step": enc_b + dec_b},
        "pct_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "encode_vectors_per_s": round(n_vec / (enc_ms / 1e3), 1),
        "encode_us": round(enc_ms * 1e3, 2),
        "attention_GBps": round(dec_b / (dec_ms / 1e3) / 1e9, 1),
        "attention_us": round(dec_ms * 1e3, 2),
        "roofline": roof,
    }
    if long_res is not None:
        line["attention_long"] = long_res
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
