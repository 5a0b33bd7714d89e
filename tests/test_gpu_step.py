"""The fused decode step (append the new token's key and value, then attend)
against the two calls it stands for, and against the oracle.

tq_decode_step is tq_encode_kv of one token per sequence followed by
tq_decode_attention with q_len 1.  The cache pools must be bit-identical to
those two calls' on the same inputs.  Fused (3-bit codes, up to 4 query heads
per KV head) the step splits each row's keys into other partial records than
the attention call (an equal share of all tiles per wave), so its output may
differ from the call's in the last bits of fp32: within 2e-5 of the row's
largest element (one bf16 step for a bf16 output); unfused it runs the two
calls' own launches and is bit-identical.  The oracle then checks the step's
output on sampled heads."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import check_decode, codebook, dev, encode_gpu, new_pools, oracle_tables
import decode_attention_tq_amd as tq

pytestmark = pytest.mark.gpu


def _setup(seed, B, Hq, Hkv, bits=3, lo=512, hi=32768, steps=2, lengths=None):
    case = synth.ragged_case(seed=seed, B=B, Hq=Hq, Hkv=Hkv, lo=lo, hi=hi, steps=steps, lengths=lengths)
    cb = codebook(bits=bits)
    kpool, vpool = new_pools(case["num_blocks"], Hkv, bits=bits)
    encode_gpu(cb, case["k"], case["v"], case["slots"], kpool, vpool, with_norms=False)
    return case, cb, kpool, vpool


def _two_calls(cb, kn, vn, slots, q, kpool, vpool, bt, cl, maxc, Hkv):
    tq.tq_encode_kv(cb, kn, vn, slots, kpool, vpool)
    return tq.tq_decode_attention(cb, q, kpool, vpool, bt, cl, maxc, Hkv)


def _same_output(out, ref, fused, rel=None):
    """Bit-identical unfused; fused, within 2e-5 of each row's largest
    magnitude (fp32 rounding of another split), or one step of a bf16 output
    (rel: another bound, for a step whose split pass is another kernel)."""
    if not fused:
        assert torch.equal(out, ref), f"outputs differ: max {float((out.float() - ref.float()).abs().max()):.3e}"
        return
    o, r = out.float(), ref.float()
    if rel is None:
        rel = 2e-5 if out.dtype == torch.float32 else 2.0 ** -7
    scale = r.abs().amax(dim=-1, keepdim=True)
    err = (o - r).abs()
    assert bool(torch.all(err <= rel * scale)), f"max err / row scale {float((err / scale.clamp_min(1e-30)).max()):.3e}"


@pytest.mark.parametrize("Hq,Hkv,bits", [(32, 8, 3), (8, 8, 3), (16, 8, 3), (64, 8, 3), (32, 8, 2)])
def test_step_is_append_then_decode(Hq, Hkv, bits):
    """Two consecutive steps of a ragged batch of 16 (lengths in [512, 4096]):
    pools and outputs equal to the separate calls' bit for bit, with one
    sequence skipping its append (slot -1, context unchanged).  Group sizes 4,
    1, 2 and 8 run fused (8: two waves per run of tiles, one head tile each);
    2-bit codes run unfused.  With 8 heads per KV head the separate attention
    call runs the 8-wave pass, which cuts the 15-bit softmax weights into
    other blocks than the step's waves: on long peaked rows their outputs
    differ by up to a few 1e-4 of the row scale, so there both are held to
    the oracle after every step and to each other within the parity bar."""
    B = 16
    case, cb, kpool, vpool = _setup(11 + Hq + bits, B, Hq, Hkv, bits=bits, hi=4096)
    ka, va = kpool.clone(), vpool.clone()
    bt = torch.from_numpy(case["table"].astype(np.int32)).cuda()
    L = case["lengths"].copy()
    ws = None
    for s in range(2):
        slots = case["new_slots"][s].copy()
        grow = np.ones(B, np.int64)
        if s == 1:
            slots[5] = -1
            grow[5] = 0
        L = L + grow
        cl = torch.from_numpy(L.astype(np.int32)).cuda()
        maxc = int(L.max())
        kn, vn = dev(case["new_k"][s], torch.bfloat16), dev(case["new_v"][s], torch.bfloat16)
        st = torch.from_numpy(slots).cuda()
        q = dev(case["q"][s], torch.bfloat16)
        ref = _two_calls(cb, kn, vn, st, q, ka, va, bt, cl, maxc, Hkv)
        if ws is None:
            need = tq.tq_decode_step_workspace_bytes(cb, B, Hq, Hkv, maxc + 1)
            ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
        out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc, workspace=ws)
        torch.cuda.synchronize()
        print(f"Hq {Hq} Hkv {Hkv} bits {bits} step {s}", flush=True)
        assert torch.equal(kpool, ka), "K pools differ"
        assert torch.equal(vpool, va), "V pools differ"
        G = Hq // Hkv
        if bits == 3 and G > 4:
            _same_output(out, ref, fused=True, rel=2e-3)
            kp, vp = kpool.cpu().numpy(), vpool.cpu().numpy()
            for o in (out, ref):
                check_decode(o.cpu().numpy(), case["q"][s], kp, vp, case["table"], L,
                             tables=oracle_tables(bits=bits), kv_heads=[0, Hkv - 1])
        else:
            _same_output(out, ref, fused=bits == 3 and G <= 4)
    if bits == 3:
        kp, vp = kpool.cpu().numpy(), vpool.cpu().numpy()
        check_decode(out.cpu().numpy(), case["q"][1], kp, vp, case["table"], L, tables=oracle_tables(bits=bits),
                     kv_heads=[0, Hkv - 1])


def test_step_fp32_and_f16_inputs_and_outputs():
    """New keys/values in fp32 with head-strided layout, an f16 query and a
    bf16 output: equal to the separate calls."""
    B, Hq, Hkv = 8, 32, 8
    case, cb, kpool, vpool = _setup(21, B, Hq, Hkv, hi=2048, steps=1)
    ka, va = kpool.clone(), vpool.clone()
    bt = torch.from_numpy(case["table"].astype(np.int32)).cuda()
    L = case["lengths"] + 1
    cl = torch.from_numpy(L.astype(np.int32)).cuda()
    maxc = int(L.max())
    # [B][Hkv][128] views into a wider buffer: token stride 2 * Hkv * 128
    buf = torch.zeros((B, 2 * Hkv, 128), dtype=torch.float32, device="cuda")
    buf[:, ::2] = dev(case["new_k"][0])
    buf[:, 1::2] = dev(case["new_v"][0])
    kn, vn = buf[:, ::2], buf[:, 1::2]
    st = torch.from_numpy(case["new_slots"][0].copy()).cuda()
    q = dev(case["q"][0], torch.float16)
    tq.tq_encode_kv(cb, kn, vn, st, ka, va)
    ref = tq.tq_decode_attention(cb, q, ka, va, bt, cl, maxc, Hkv, out_dtype=torch.bfloat16)
    out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(kpool, ka) and torch.equal(vpool, va)
    _same_output(out, ref, fused=True)


def test_step_short_and_empty_sequences():
    """Context lengths 1 (the new token alone), 16, 17 and 0 with a skipped
    append: the plan gives such sequences no range or one short one."""
    B, Hq, Hkv = 4, 32, 8
    case, cb, kpool, vpool = _setup(31, B, Hq, Hkv, steps=1, lengths=[0, 15, 16, 300])
    ka, va = kpool.clone(), vpool.clone()
    bt = torch.from_numpy(case["table"].astype(np.int32)).cuda()
    slots = case["new_slots"][0].copy()
    L = case["lengths"] + 1
    slots[3] = -1
    L[3] = 0
    cl = torch.from_numpy(L.astype(np.int32)).cuda()
    maxc = int(L.max())
    kn, vn = dev(case["new_k"][0], torch.bfloat16), dev(case["new_v"][0], torch.bfloat16)
    st = torch.from_numpy(slots).cuda()
    q = dev(case["q"][0], torch.bfloat16)
    ref = _two_calls(cb, kn, vn, st, q, ka, va, bt, cl, maxc, Hkv)
    out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc)
    torch.cuda.synchronize()
    assert torch.equal(kpool, ka) and torch.equal(vpool, va)
    _same_output(out, ref, fused=True)
    o = out.cpu().numpy()
    assert not np.any(o[3])                      # no key at all: zero output
    check_decode(o, case["q"][0], kpool.cpu().numpy(), vpool.cpu().numpy(), case["table"], L)


def test_step_decode_batch_full_size_sampled():
    """The decode-step workload at full size: 16 sequences, log-uniform
    lengths in [512, 32768], 32 query and 8 KV heads.  Equal to the separate
    calls everywhere; the oracle checks sampled KV heads."""
    B, Hq, Hkv = 16, 32, 8
    case, cb, kpool, vpool = _setup(3, B, Hq, Hkv, steps=1)
    ka, va = kpool.clone(), vpool.clone()
    bt = torch.from_numpy(case["table"].astype(np.int32)).cuda()
    L = case["lengths"] + 1
    cl = torch.from_numpy(L.astype(np.int32)).cuda()
    maxc = int(L.max())
    kn, vn = dev(case["new_k"][0], torch.bfloat16), dev(case["new_v"][0], torch.bfloat16)
    st = torch.from_numpy(case["new_slots"][0].copy()).cuda()
    q = dev(case["q"][0], torch.bfloat16)
    ref = _two_calls(cb, kn, vn, st, q, ka, va, bt, cl, maxc, Hkv)
    out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc)
    torch.cuda.synchronize()
    assert torch.equal(kpool, ka) and torch.equal(vpool, va)
    _same_output(out, ref, fused=True)
    check_decode(out.cpu().numpy(), case["q"][0], kpool.cpu().numpy(), vpool.cpu().numpy(), case["table"], L,
                 kv_heads=[2])


def test_step_more_than_64_sequences_and_large_appends():
    """80 sequences (the plan's sequence blocks of 64 lanes: the table,
    the runs per die and the operand groups span two blocks), then 140
    sequences x 8 KV heads = 1,120 appended vectors, past the one-wave
    append (the step runs the tiled encoder and the attention call's own
    launches).  Pools and outputs equal to the separate calls; the oracle
    checks sampled heads."""
    for B, hi in ((80, 3000), (140, 1500)):
        Hq, Hkv = 32, 8
        case, cb, kpool, vpool = _setup(41 + B, B, Hq, Hkv, lo=1, hi=hi, steps=1)
        ka, va = kpool.clone(), vpool.clone()
        bt = torch.from_numpy(case["table"].astype(np.int32)).cuda()
        L = case["lengths"] + 1
        cl = torch.from_numpy(L.astype(np.int32)).cuda()
        maxc = int(L.max())
        kn, vn = dev(case["new_k"][0], torch.bfloat16), dev(case["new_v"][0], torch.bfloat16)
        st = torch.from_numpy(case["new_slots"][0].copy()).cuda()
        q = dev(case["q"][0], torch.bfloat16)
        ref = _two_calls(cb, kn, vn, st, q, ka, va, bt, cl, maxc, Hkv)
        out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc)
        torch.cuda.synchronize()
        print(f"B {B}: step done", flush=True)
        assert torch.equal(kpool, ka) and torch.equal(vpool, va)
        _same_output(out, ref, fused=B * Hkv <= 1024)
        check_decode(out.cpu().numpy(), case["q"][0], kpool.cpu().numpy(), vpool.cpu().numpy(), case["table"], L,
                     kv_heads=[1, 6])


def test_step_eight_consecutive_steps_one_workspace():
    """Eight fused steps in a row with one workspace (uninitialised at the
    first call), new queries every step: after every step the pools are
    bit-identical to the separate calls' and the output within rounding of
    theirs; the oracle checks the last step."""
    B, Hq, Hkv, S = 16, 32, 8, 8
    case, cb, kpool, vpool = _setup(61, B, Hq, Hkv, hi=6000, steps=S)
    ka, va = kpool.clone(), vpool.clone()
    bt = torch.from_numpy(case["table"].astype(np.int32)).cuda()
    L = case["lengths"].copy()
    ws = torch.empty(tq.tq_decode_step_workspace_bytes(cb, B, Hq, Hkv, int(L.max()) + S), dtype=torch.uint8,
                     device="cuda")
    for s in range(S):
        L = L + 1
        cl = torch.from_numpy(L.astype(np.int32)).cuda()
        maxc = int(L.max())
        kn, vn = dev(case["new_k"][s], torch.bfloat16), dev(case["new_v"][s], torch.bfloat16)
        st = torch.from_numpy(case["new_slots"][s].copy()).cuda()
        q = dev(case["q"][s], torch.bfloat16)
        ref = _two_calls(cb, kn, vn, st, q, ka, va, bt, cl, maxc, Hkv)
        out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc, workspace=ws)
        torch.cuda.synchronize()
        print(f"step {s} done", flush=True)
        assert torch.equal(kpool, ka) and torch.equal(vpool, va), f"pools differ after step {s}"
        _same_output(out, ref, fused=True)
    check_decode(out.cpu().numpy(), case["q"][S - 1], kpool.cpu().numpy(), vpool.cpu().numpy(), case["table"], L,
                 kv_heads=[0, 5])


def _device_cache_case(seed, lengths, Hq=32, Hkv=8):
    """Pools holding ``lengths`` cached tokens per sequence, drawn on the
    device with the GQA recipe (synth.kv_tensor_device) and encoded; room
    for one more token each; new tokens and queries for one step.  The
    oracle checks read the encoded pages, so the raw cache stays on the
    device."""
    rng = np.random.default_rng(seed)
    L = np.asarray(lengths, np.int64)
    B = len(L)
    table, nb = synth.block_tables(rng, L + 1)
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv, seed=seed)
    slots = np.concatenate([synth.slots_for(table, b, np.arange(L[b])) for b in range(B)])
    kt = synth.kv_tensor_device(seed, len(slots), Hkv, "cuda")
    vt = synth.kv_tensor_device(seed + 1, len(slots), Hkv, "cuda")
    tq.tq_encode_kv(cb, kt, vt, torch.from_numpy(slots).cuda(), kpool, vpool)
    del kt, vt
    new_slots = np.array([synth.slots_for(table, b, [L[b]])[0] for b in range(B)], np.int64)
    kn = synth.kv_tensor_device(seed + 2, B, Hkv, "cuda")
    vn = synth.kv_tensor_device(seed + 3, B, Hkv, "cuda")
    q = rng.standard_normal((B, 1, Hq, 128)).astype(np.float32)
    return cb, kpool, vpool, table, L + 1, new_slots, kn, vn, q


@pytest.mark.parametrize("name,lengths,Hq", [
    ("64 sequences of one tile", [1 + 2 * b for b in range(64)], 32),
    ("two long sequences", [131071, 99999], 32),
    ("more tiles than one round of waves", [40000] * 8 + [30000] * 8, 32),
    ("64 sequences of one tile, 8 heads per KV head", [1 + 2 * b for b in range(64)], 64),
    ("more tiles than one round of waves, 6 heads per KV head", [40000] * 8 + [30000] * 8, 48),
])
def test_step_stream_plan_extremes(name, lengths, Hq):
    """The step's split plan at its ends: 64 one-tile sequences (one tile
    per wave, one wave per group); two sequences of 131,072 and 100,000
    tokens (8 tiles per wave, a group spread over hundreds of waves); 16
    sequences of 30,000-40,000 tokens, 35,072 tiles (16 tiles per wave, more
    workgroups than run at once).  Pools bit-identical to the separate
    calls, outputs within rounding of theirs, the oracle on sampled
    sequences and KV heads.  With 6 and 8 query heads per KV head the waves
    go in pairs (one head tile each) over the same runs of tiles."""
    Hkv = 8
    cb, kpool, vpool, table, L, new_slots, kn, vn, qn = _device_cache_case(71 + len(lengths), lengths, Hq, Hkv)
    ka, va = kpool.clone(), vpool.clone()
    bt = torch.from_numpy(table.astype(np.int32)).cuda()
    cl = torch.from_numpy(L.astype(np.int32)).cuda()
    maxc = int(L.max())
    st = torch.from_numpy(new_slots).cuda()
    q = dev(qn, torch.bfloat16)
    ref = _two_calls(cb, kn, vn, st, q, ka, va, bt, cl, maxc, Hkv)
    out = tq.tq_decode_step(cb, kn, vn, st, q, kpool, vpool, bt, cl, maxc)
    torch.cuda.synchronize()
    print(f"{name}: step done", flush=True)
    assert torch.equal(kpool, ka) and torch.equal(vpool, va)
    # 5 to 8 heads: the separate call runs the 8-wave pass (other weight
    # blocks), so the two are held to the oracle and to the parity bar
    _same_output(out, ref, fused=True, rel=2e-3 if Hq // Hkv > 4 else None)
    kp, vp = kpool.cpu().numpy(), vpool.cpu().numpy()
    q64 = q.float().cpu().numpy()
    seqs = [0, len(L) - 1]
    check_decode(out.cpu().numpy(), q64, kp, vp, table, L, seqs=seqs, kv_heads=[1, Hkv - 2])
