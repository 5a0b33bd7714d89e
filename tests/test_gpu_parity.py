"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases are checked element by element; the full-size workloads, in the
launch configuration the benchmark uses, are checked on sampled heads,
positions and query rows.  Tolerances: see gpu_helpers."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (OUT_RTOL, assert_rows_close, check_decode, check_encoded_sequence, codebook,
                         decode_gpu, dev, encode_gpu, new_pools, oracle_tables, rel_rows)
from oracle import decode_paged_hot
import decode_attention_tq_amd as tq

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


def test_single_head_fp32_1024_tokens():
    case = synth.single_head_case(seed=1, T=1024)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 1)
    norms = encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, dtype=torch.float32)
    kp, vp = _np(kpool), _np(vpool)
    stats = {}
    check_encoded_sequence(case["k"], case["v"], kp, vp, case["table"][0], np.arange(1024), norms,
                           stats=stats)
    print("ambiguous codes:", stats)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 1,
                     q_dtype=torch.float32)
    err = check_decode(out, case["q"], kp, vp, case["table"], case["context_lens"])
    print("max rel err", err.max())


@pytest.mark.parametrize("T", [1000, 8192])
def test_gqa_32q_8kv(T):
    case = synth.gqa_case(seed=2, T=T, Hq=32, Hkv=8)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 8)
    norms = encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool)
    kp, vp = _np(kpool), _np(vpool)
    check_encoded_sequence(case["k"], case["v"], kp, vp, case["table"][0], np.arange(T), norms)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 8)
    err = check_decode(out, case["q"], kp, vp, case["table"], case["context_lens"])
    print("max rel err", err.max())


def test_ragged_batch_with_appends():
    # 16 sequences, log-uniform lengths in [512, 32768], random block table,
    # then two decode steps that each append and encode one token per sequence.
    case = synth.ragged_case(seed=3, B=16, Hq=32, Hkv=8, steps=2)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 8)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    L = case["lengths"].copy()
    starts = np.concatenate([[0], np.cumsum(L)])
    for step in range(2):
        norms = encode_gpu(cb, case["new_k"][step], case["new_v"][step], case["new_slots"][step],
                           kpool, vpool)
        L = L + 1
        kp, vp = _np(kpool), _np(vpool)
        for b in (0, 7):       # sampled sequences: whole history + the appended tokens
            hist_k = np.concatenate([case["k"][starts[b]:starts[b + 1]]] +
                                    [case["new_k"][s][b:b + 1] for s in range(step + 1)])
            hist_v = np.concatenate([case["v"][starts[b]:starts[b + 1]]] +
                                    [case["new_v"][s][b:b + 1] for s in range(step + 1)])
            check_encoded_sequence(hist_k, hist_v, kp, vp, case["table"][b], np.arange(L[b]), None)
        out = decode_gpu(cb, case["q"][step], kpool, vpool, case["table"], L.astype(np.int32), 8)
        err = check_decode(out, case["q"][step], kp, vp, case["table"], L, kv_heads=[0, 5])
        print("step", step, "max rel err", err.max())


def test_long_context_131072_split_k():
    case = synth.gqa_case(seed=4, T=131072, Hq=32, Hkv=4)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 4, fill="zeros")
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    kp, vp = _np(kpool), _np(vpool)
    pos = np.r_[0:2048, 131072 - 2048:131072]
    check_encoded_sequence(case["k"][pos], case["v"][pos], kp, vp, case["table"][0], pos, None)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 4)
    err = check_decode(out, case["q"], kp, vp, case["table"], case["context_lens"], kv_heads=[0, 3])
    print("max rel err", err.max())


@pytest.mark.parametrize("cached,new", [(300, 37), (32768, 2048)])
def test_chunked_prefill_causal(cached, new):
    T = cached + new
    case = synth.gqa_case(seed=5, T=T, Hq=32, Hkv=8, q_len=new)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 8)
    encode_gpu(cb, case["k"][:cached], case["v"][:cached], case["slots"][:cached], kpool, vpool,
               with_norms=False)
    norms = encode_gpu(cb, case["k"][cached:], case["v"][cached:], case["slots"][cached:],
                       kpool, vpool)
    kp, vp = _np(kpool), _np(vpool)
    sample = np.arange(T) if T < 1000 else np.r_[0:256, cached - 16:T]
    check_encoded_sequence(case["k"][sample], case["v"][sample], kp, vp, case["table"][0], sample, None)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 8)
    sub = {} if T < 1000 else dict(kv_heads=[0, 7], q_positions=[0, 1, new // 2, new - 1])
    err = check_decode(out, case["q"], kp, vp, case["table"], case["context_lens"], **sub)
    print("max rel err", err.max())


def test_edge_cases_encode():
    cb = codebook()
    rng = np.random.default_rng(6)
    T, H = 40, 2
    k = synth.kv_tensor(rng, T, H)
    v = synth.kv_tensor(rng, T, H)
    k[3] = 0.0                    # zero key vector
    v[4] = 0.0                    # zero value vector
    table = np.array([[2, 0, 1]], dtype=np.int32)
    slots = synth.slots_for(table, 0, np.arange(T))
    slots[[7, 30]] = -1           # skipped tokens keep their old bytes
    kpool, vpool = new_pools(3, H, seed=1)
    before_k, before_v = _np(kpool), _np(vpool)
    norms = encode_gpu(cb, k, v, slots, kpool, vpool)
    kp, vp = _np(kpool), _np(vpool)
    keep = np.array([j for j in range(T) if slots[j] >= 0])
    check_encoded_sequence(k[keep], v[keep], kp, vp, table[0], keep, norms[keep])
    from oracle.pages import read_k_tokens_fast, read_v_tokens_fast
    for h in range(H):
        for j in (7, 30):
            a = read_k_tokens_fast(kp, table[0], T, h)
            b = read_k_tokens_fast(before_k, table[0], T, h)
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x[j], y[j])
            a = read_v_tokens_fast(vp, table[0], T, h)
            b = read_v_tokens_fast(before_v, table[0], T, h)
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x[j], y[j])
        codes = read_k_tokens_fast(kp, table[0], T, h)[0]
        np.testing.assert_array_equal(codes[3], np.full(128, 3))
    assert np.all(norms[3, :, 0] == 0) and np.all(norms[4, :, 2] == 0)
    # zero tokens: a no-op
    e = torch.empty((0, H, 128), dtype=torch.bfloat16, device="cuda")
    import decode_attention_tq_amd as tq
    tq.tq_encode_kv(cb, e, e, torch.empty(0, dtype=torch.int64, device="cuda"), kpool, vpool)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(kpool), kp)


def test_partial_pages_across_calls_and_fp16_input():
    # tokens of one page arrive in several calls (the atomic merge path)
    cb = codebook()
    rng = np.random.default_rng(7)
    T, H = 70, 3
    k = synth.kv_tensor(rng, T, H, bf16=False).astype(np.float16).astype(np.float32)
    v = synth.kv_tensor(rng, T, H, bf16=False).astype(np.float16).astype(np.float32)
    table = np.array([[4, 1, 3, 0, 2]], dtype=np.int32)
    slots = synth.slots_for(table, 0, np.arange(T))
    kpool, vpool = new_pools(5, H, seed=2)
    order = rng.permutation(T)
    for chunk in np.array_split(order, 7):
        sl = np.full(T, -1, dtype=np.int64)
        sl[chunk] = slots[chunk]
        encode_gpu(cb, k, v, sl, kpool, vpool, dtype=torch.float16, with_norms=False)
    check_encoded_sequence(k, v, _np(kpool), _np(vpool), table[0], np.arange(T), None)


def test_decode_edge_cases_and_dtypes():
    cb = codebook()
    case = synth.ragged_case(seed=8, B=5, Hq=16, Hkv=1, lengths=[0, 1, 15, 16, 700])
    kpool, vpool = new_pools(case["num_blocks"], 1)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    kp, vp = _np(kpool), _np(vpool)
    L = case["lengths"].astype(np.int32)
    q = case["q"][0]
    for qd, od in ((torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16),
                   (torch.float16, torch.float16)):
        out = decode_gpu(cb, q, kpool, vpool, case["table"], L, 1, q_dtype=qd, out_dtype=od)
        tol = 2e-3 if od == torch.float32 else 1e-2
        qq = dev(q, qd).float().cpu().numpy()
        check_decode(out, qq, kp, vp, case["table"], L, rtol=tol)
    assert np.all(out[0] == 0)                       # empty context -> zeros
    # a custom softmax scale
    out = decode_gpu(cb, q, kpool, vpool, case["table"], L, 1, scale=0.3)
    check_decode(out, q, kp, vp, case["table"], L, scale=0.3)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (16, 2)])
def test_matrix_core_pass_query_dtypes(Hq, Hkv):
    """The matrix-core pass forms its query operands from raw q words: fp16
    and fp32 queries (elements in both halves of a word) with four and eight
    heads per KV head, ragged contexts including an empty one."""
    cb = codebook()
    case = synth.ragged_case(seed=13, B=3, Hq=Hq, Hkv=Hkv, lengths=[0, 300, 1300])
    kpool, vpool = new_pools(case["num_blocks"], Hkv)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    kp, vp = _np(kpool), _np(vpool)
    L = case["lengths"].astype(np.int32)
    q = case["q"][0]
    for qd in (torch.float16, torch.float32):
        out = decode_gpu(cb, q, kpool, vpool, case["table"], L, Hkv, q_dtype=qd)
        qq = dev(q, qd).float().cpu().numpy()
        check_decode(out, qq, kp, vp, case["table"], L)
        assert np.all(out[0] == 0)


def test_split_invariance_permutation_invariance_determinism():
    cb = codebook()
    case = synth.gqa_case(seed=9, T=3000, Hq=16, Hkv=2)
    kpool, vpool = new_pools(case["num_blocks"], 2)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    outs = [decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 2,
                       tokens_per_split=tps) for tps in (0, 256, 512, 3072)]
    for o in outs[1:]:
        assert rel_rows(o, outs[0].astype(np.float64)).max() < 1e-5
    again = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 2)
    np.testing.assert_array_equal(again, outs[0])
    # relabel physical blocks: identical results
    nb = case["num_blocks"]
    perm = np.random.default_rng(0).permutation(nb)
    k2 = torch.empty_like(kpool)
    v2 = torch.empty_like(vpool)
    k2[torch.from_numpy(perm).cuda()] = kpool
    v2[torch.from_numpy(perm).cuda()] = vpool
    out2 = decode_gpu(cb, case["q"], k2, v2, perm[case["table"]], case["context_lens"], 2)
    np.testing.assert_array_equal(out2, outs[0])
    # encode is deterministic too
    kp3, vp3 = new_pools(nb, 2)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kp3, vp3, with_norms=False)
    np.testing.assert_array_equal(_np(kp3), _np(kpool))
    np.testing.assert_array_equal(_np(vp3), _np(vpool))


def test_caller_supplied_qjl_matrix():
    import decode_attention_tq_amd as tq
    S = np.random.default_rng(10).standard_normal((128, 128)).astype(np.float32)
    cb = tq.tq_codebook_init(128, 3, 0, qjl_host=S, device="cuda")
    c32, t32, _ = oracle_tables()
    case = synth.gqa_case(seed=10, T=500, Hq=8, Hkv=2)
    kpool, vpool = new_pools(case["num_blocks"], 2)
    norms = encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool)
    kp, vp = _np(kpool), _np(vpool)
    check_encoded_sequence(case["k"], case["v"], kp, vp, case["table"][0], np.arange(500), norms,
                           tables=(c32, t32, S))
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 2)
    check_decode(out, case["q"], kp, vp, case["table"], case["context_lens"], tables=(c32, t32, S))


@pytest.mark.parametrize("Hq,Hkv,T", [(4, 4, 777), (8, 4, 777), (8, 2, 131), (16, 2, 131)])
def test_small_groups(Hq, Hkv, T):
    """One and two query heads per KV head (unused operand rows), a context
    shorter than one 128-token tile, and eight heads per KV head (the pass
    whose waves split into scoring and value roles) over a partial tile."""
    case = synth.gqa_case(seed=11, T=T, Hq=Hq, Hkv=Hkv)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], Hkv)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], Hkv)
    check_decode(out, case["q"], _np(kpool), _np(vpool), case["table"], case["context_lens"])


@pytest.mark.parametrize("Hkv", [8, 4])
def test_running_maximum_moves_along_the_sequence(Hkv):
    """Key norms ramp up 8x along the context with softmax scale 0.25: the
    maximum log2-score grows from about 40 to about 350, so later tiles
    overtake the running maximum by more than the rescale threshold (64)
    several times; the output must still match (4 and 8 heads per KV head)."""
    T = 4096
    case = synth.gqa_case(seed=12, T=T, Hq=32, Hkv=Hkv)
    ramp = (1.0 + 7.0 * np.arange(T) / T)[:, None, None]
    k = synth.round_to_bf16(case["k"] * ramp)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], Hkv)
    encode_gpu(cb, k, case["v"], case["slots"], kpool, vpool, with_norms=False)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], Hkv,
                     scale=0.25, tokens_per_split=4096)
    err = check_decode(out, case["q"], _np(kpool), _np(vpool), case["table"],
                       case["context_lens"], scale=0.25)
    print("max rel err", err.max())


@pytest.mark.parametrize("q_len,Hq,Hkv", [(2, 32, 8), (3, 4, 2), (8, 8, 8), (4, 32, 8), (3, 32, 4),
                                         (8, 32, 4), (3, 16, 1), (8, 32, 8), (32, 8, 8), (5, 24, 8)])
def test_multi_token_verify(q_len, Hq, Hkv):
    """Multi-token verify decode (speculative or multi-token prediction): 2 to
    32 new queries per sequence over a compressed cache, each causal over the
    cache plus the verified tokens before it, batched sequences of ragged
    length (the first as long as the block).  Up to 8 query rows (positions x
    heads) per KV head run the balanced plan's launch (4, 6 and 8 rows
    here); 9 to 32 rows the stream plan, one wave per head tile of four rows
    (12, 24, 32 and 15 rows here, with 1, 3, 4 and 8 heads per KV head);
    longer blocks take the prefill pass."""
    rng = np.random.default_rng(20 + q_len)
    lens = np.array([q_len, 700, 2300], dtype=np.int64)
    table, nb = synth.block_tables(rng, lens)
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv)
    for b in range(len(lens)):
        k = synth.kv_tensor(rng, int(lens[b]), Hkv)
        v = synth.kv_tensor(rng, int(lens[b]), Hkv)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    q = synth.queries(rng, len(lens), q_len, Hq)
    out = decode_gpu(cb, q, kpool, vpool, table, lens.astype(np.int32), Hkv)
    check_decode(out, q, _np(kpool), _np(vpool), table, lens.astype(np.int32))


def test_verify_blocks_on_the_stream_plan_sweep():
    """Seeded sweep of verify blocks that run the stream plan (9 to 32 query
    rows per KV head, one wave per head tile of four (position, head) rows):
    random group sizes (1 to 8), block lengths and KV head counts over
    ragged batches holding a sequence exactly as long as the block, one
    shorter than a tile and one of several tiles with a ragged tail; every
    row against the oracle."""
    rng = np.random.default_rng(91)
    cb = codebook()
    done = 0
    while done < 8:
        G = int(rng.integers(1, 9))
        Hkv = int(rng.choice([1, 2, 4]))
        q_len = int(rng.integers(2, 4 * (8 // G) + 1))  # at most four launches' worth of positions
        if G * q_len <= 8:
            continue
        lens = np.array([q_len, int(rng.integers(q_len, 128)), int(rng.integers(300, 3000))], dtype=np.int64)
        table, nb = synth.block_tables(rng, lens)
        kpool, vpool = new_pools(nb, Hkv)
        for b in range(len(lens)):
            k = synth.kv_tensor(rng, int(lens[b]), Hkv)
            v = synth.kv_tensor(rng, int(lens[b]), Hkv)
            encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
        q = synth.queries(rng, len(lens), q_len, G * Hkv)
        print(f"G {G} Hkv {Hkv} q_len {q_len} lens {lens.tolist()}", flush=True)
        out = decode_gpu(cb, q, kpool, vpool, table, lens.astype(np.int32), Hkv)
        check_decode(out, q, _np(kpool), _np(vpool), table, lens.astype(np.int32))
        done += 1


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (32, 4), (32, 2)])
def test_prefill_groups_batches_and_splits(Hq, Hkv):
    """Several queries per sequence for every supported group size (1, 2, 8,
    16 query heads per KV head): two sequences of different lengths, a query
    count that leaves a partial block of positions, and chunks of 256 keys
    that cut through the causal boundary."""
    rng = np.random.default_rng(11 + Hq // Hkv)
    lens = np.array([200, 517], dtype=np.int64)
    q_len = 21
    table, nb = synth.block_tables(rng, lens)
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv)
    for b in range(len(lens)):
        k = synth.kv_tensor(rng, int(lens[b]), Hkv)
        v = synth.kv_tensor(rng, int(lens[b]), Hkv)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    q = synth.queries(rng, len(lens), q_len, Hq)
    kp, vp = _np(kpool), _np(vpool)
    cl = lens.astype(np.int32)
    outs = []
    for tps in (0, 256):
        out = decode_gpu(cb, q, kpool, vpool, table, cl, Hkv, tokens_per_split=tps)
        check_decode(out, q, kp, vp, table, cl)
        outs.append(out)
    # a different chunking changes only the rounding of the combine
    assert np.abs(outs[0] - outs[1]).max() <= 1e-4 * max(1.0, np.abs(outs[0]).max())


@pytest.mark.parametrize("Hq,Hkv", [(12, 4), (15, 3), (24, 4), (28, 4), (24, 2)])
def test_any_group_size(Hq, Hkv):
    """Group sizes that are not powers of two (3, 5, 6, 7 and 12 query heads
    per KV head, e.g. 28q/4kv): single-query decode (matrix-core pass for up
    to 8 heads, vector pass above), a 3-token verify block, a 21-token
    chunked prefill block and the exact hot window, each against the oracle
    on two ragged sequences."""
    G = Hq // Hkv
    rng = np.random.default_rng(60 + G)
    lens = np.array([700, 2300], dtype=np.int64)
    table, nb = synth.block_tables(rng, lens)
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv)
    for b in range(len(lens)):
        k = synth.kv_tensor(rng, int(lens[b]), Hkv)
        v = synth.kv_tensor(rng, int(lens[b]), Hkv)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    kp, vp = _np(kpool), _np(vpool)
    cl = lens.astype(np.int32)
    for q_len in (1, 3, 21):
        q = synth.queries(rng, len(lens), q_len, Hq)
        out = decode_gpu(cb, q, kpool, vpool, table, cl, Hkv)
        err = check_decode(out, q, kp, vp, table, cl)
        print("G", G, "q_len", q_len, "max rel err", err.max())
    W, hot_max = np.array([77, 300], dtype=np.int32), 300
    hk = torch.from_numpy(synth.kv_tensor(rng, 2 * hot_max, Hkv).reshape(2, hot_max, Hkv, 128)).to(torch.bfloat16)
    hv = torch.from_numpy(synth.kv_tensor(rng, 2 * hot_max, Hkv).reshape(2, hot_max, Hkv, 128)).to(torch.bfloat16)
    q = synth.queries(rng, len(lens), 1, Hq)
    out = tq.tq_decode_attention_hot(
        cb, dev(q, torch.bfloat16), kpool, vpool, torch.from_numpy(table).cuda(), torch.from_numpy(cl).cuda(),
        int(lens.max()), Hkv, hk.cuda(), hv.cuda(), torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    c32, _, S = oracle_tables()
    ref = decode_paged_hot(np.asarray(q, np.float64), kp, vp, table, lens, hk.double().numpy(), hv.double().numpy(),
                           W, c32, S)
    assert_rows_close(out.float().cpu().numpy(), ref)


@pytest.mark.parametrize("Hq,Hkv,hot_dtype", [(32, 8, torch.bfloat16), (16, 16, torch.float16),
                                             (32, 4, torch.float32), (32, 2, torch.bfloat16)])
def test_hot_window(Hq, Hkv, hot_dtype):
    """Decode over a compressed history followed by an exact hot window of
    recent tokens, one softmax over both: ragged histories (one empty) and
    windows (one empty, one of 2,048 tokens, several 64-token chunks and a
    ragged last one), a sequence with no key at all (zero output), 1 to 16
    query heads per KV head, window tokens in bf16, f16 and f32."""
    rng = np.random.default_rng(40 + Hq // Hkv)
    lens = np.array([0, 700, 2300, 5, 0], dtype=np.int64)
    hot = np.array([300, 0, 2048, 77, 0], dtype=np.int32)
    B, hot_max = len(lens), 2048
    table, nb = synth.block_tables(rng, np.maximum(lens, 1))
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv)
    for b in range(B):
        if lens[b] == 0:
            continue
        k = synth.kv_tensor(rng, int(lens[b]), Hkv)
        v = synth.kv_tensor(rng, int(lens[b]), Hkv)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    hk = torch.from_numpy(synth.kv_tensor(rng, B * hot_max, Hkv).reshape(B, hot_max, Hkv, 128)).to(hot_dtype)
    hv = torch.from_numpy(synth.kv_tensor(rng, B * hot_max, Hkv).reshape(B, hot_max, Hkv, 128)).to(hot_dtype)
    q = synth.queries(rng, B, 1, Hq)
    out = tq.tq_decode_attention_hot(
        cb, dev(q, torch.bfloat16), kpool, vpool, torch.from_numpy(table).cuda(),
        torch.from_numpy(lens.astype(np.int32)).cuda(), int(lens.max()), Hkv,
        hk.cuda(), hv.cuda(), torch.from_numpy(hot).cuda())
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    c32, _, S = oracle_tables()
    ref = decode_paged_hot(np.asarray(q, np.float64), _np(kpool), _np(vpool), table, lens, hk.double().numpy(),
                           hv.double().numpy(), hot, c32, S)
    assert_rows_close(out, ref)
    assert np.all(out[4] == 0)  # no key at all


def test_hot_window_empty_is_the_plain_call():
    """With no window (hot_max 0, null window pointers) the call is the plain
    decode launch sequence: bit-identical output."""
    case = synth.gqa_case(seed=13, T=1500, Hq=32, Hkv=8)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 8)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    q = dev(case["q"], torch.bfloat16)
    bt = torch.from_numpy(case["table"]).cuda()
    cl = torch.from_numpy(case["context_lens"]).cuda()
    T = int(case["context_lens"].max())
    plain = tq.tq_decode_attention(cb, q, kpool, vpool, bt, cl, T, 8)
    empty = torch.empty((1, 0, 8, 128), dtype=torch.bfloat16, device="cuda")
    hot = tq.tq_decode_attention_hot(cb, q, kpool, vpool, bt, cl, T, 8, empty, empty,
                                     torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(plain, hot)


def test_hot_window_bench_size_sampled():
    """The hot-window decode at the size bench.py --hot-window-only times
    (8,192 compressed tokens + a 2,048-token bf16 window, 32q/8kv), checked
    on two sampled KV heads (eight query heads)."""
    case = synth.gqa_case(seed=14, T=8192, Hq=32, Hkv=8)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 8)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    rng = np.random.default_rng(15)
    W = 2048
    hk = torch.from_numpy(synth.kv_tensor(rng, W, 8).reshape(1, W, 8, 128)).to(torch.bfloat16)
    hv = torch.from_numpy(synth.kv_tensor(rng, W, 8).reshape(1, W, 8, 128)).to(torch.bfloat16)
    hl = np.array([W], dtype=np.int32)
    out = tq.tq_decode_attention_hot(
        cb, dev(case["q"], torch.bfloat16), kpool, vpool, torch.from_numpy(case["table"]).cuda(),
        torch.from_numpy(case["context_lens"]).cuda(), 8192, 8, hk.cuda(), hv.cuda(), torch.from_numpy(hl).cuda())
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    c32, _, S = oracle_tables()
    ref = decode_paged_hot(np.asarray(case["q"], np.float64), _np(kpool), _np(vpool), case["table"],
                           case["context_lens"], hk.double().numpy(), hv.double().numpy(), hl, c32, S,
                           kv_heads=[0, 5])
    err = assert_rows_close(out, ref)
    assert err.size == 8


@pytest.mark.parametrize("q_len", [2, 8])
def test_multi_token_verify_bench_size_sampled(q_len):
    """Multi-token verify at the size bench.py --verify-only times (32,768
    compressed tokens, 32q/8kv; one and four launches), checked on two
    sampled KV heads and every new position."""
    case = synth.gqa_case(seed=16 + q_len, T=32768, Hq=32, Hkv=8, q_len=q_len)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], 8)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], 8)
    err = check_decode(out, case["q"], _np(kpool), _np(vpool), case["table"], case["context_lens"],
                       kv_heads=[2, 7])
    assert err.size == 2 * 4 * q_len


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (32, 8)])
def test_largest_chunk_of_the_matrix_core_pass(Hq, Hkv):
    """A caller's tokens_per_split of 8,192 (64 tiles of 128 tokens, the
    largest chunk the pass keeps block ids for) followed by a ragged second
    chunk; 8 and 4 query heads per KV head, checked on two sampled KV heads."""
    T = 8192 + 700
    case = synth.gqa_case(seed=30 + Hkv, T=T, Hq=Hq, Hkv=Hkv)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], Hkv)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    out = decode_gpu(cb, case["q"], kpool, vpool, case["table"], case["context_lens"], Hkv,
                     tokens_per_split=8192)
    check_decode(out, case["q"], _np(kpool), _np(vpool), case["table"], case["context_lens"],
                 kv_heads=[0, Hkv - 1])


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (32, 8), (40, 8), (64, 8)])
def test_last_tile_with_a_few_tokens(Hq, Hkv):
    """Sequences whose last 128-token tile holds 2, 3 or 15 tokens, with 1, 2,
    4, 5 and 8 query heads per KV head and two chunk sizes: the masked slots of
    that tile (pages re-read past the end, slots never written) must get no
    weight.  Element-wise against the oracle on every head."""
    lengths = [643, 1154, 3343, 836, 1249, 2, 130, 3]
    case = synth.ragged_case(seed=17, B=len(lengths), Hq=Hq, Hkv=Hkv, steps=1, lengths=lengths)
    cb = codebook()
    kpool, vpool = new_pools(case["num_blocks"], Hkv)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    L = case["lengths"]
    kp, vp = _np(kpool), _np(vpool)
    for tps in (0, 2048):
        out = decode_gpu(cb, case["q"][0], kpool, vpool, case["table"], L.astype(np.int32), Hkv,
                         tokens_per_split=tps)
        err = check_decode(out, case["q"][0], kp, vp, case["table"], L)
        print(f"Hq {Hq} tps {tps}: max rel err {err.max():.3e}")
