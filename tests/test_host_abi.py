"""Host-side checks of the C ABI: the library loads, exports everything tq.h
declares, reproduces the oracle's codebook and QJL matrix, and rejects bad
arguments before touching the device.  No GPU needed: every call here either
is host-only or fails validation before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_tq_amd as tq
from oracle import codebook_fp32, gaussian_matrix

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call using it is rejected on the host


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert "tq_encode_kv" in names and "tq_decode_attention" in names
    for n in names:
        assert hasattr(tq._lib, n), n
    assert sorted(tq.EXPORTED) == names


def test_codebook_matches_oracle_within_one_ulp():
    for bits in (1, 2, 3, 4):
        c, t = tq.tq_codebook_compute(128, bits)
        oc, ot = codebook_fp32(128, bits)
        ulps_c = np.abs(c.view(np.int32).astype(np.int64) - oc.view(np.int32).astype(np.int64))
        ulps_t = np.abs(t.view(np.int32).astype(np.int64) - ot.view(np.int32).astype(np.int64))
        assert ulps_c.max() <= 1 and ulps_t.max() <= 1, bits
    c, t = tq.tq_codebook_compute(128, 3)
    oc, ot = codebook_fp32(128, 3)
    np.testing.assert_array_equal(c, oc)   # identical in practice
    np.testing.assert_array_equal(t, ot)


@pytest.mark.parametrize("seed", [0, 42, 2 ** 63 + 5])
def test_qjl_matrix_bit_identical_to_oracle(seed):
    np.testing.assert_array_equal(tq.tq_qjl_matrix(seed, 128, 128), gaussian_matrix(seed, 128, 128))
    np.testing.assert_array_equal(tq.tq_qjl_matrix(seed, 3, 5), gaussian_matrix(seed, 3, 5))


def test_host_helper_errors():
    assert tq._lib.tq_codebook_compute(128, 0, FAKE, FAKE) == tq.TQ_ERR_UNSUPPORTED
    assert tq._lib.tq_codebook_compute(128, 3, None, FAKE) == tq.TQ_ERR_INVALID_ARGUMENT
    assert tq._lib.tq_qjl_matrix(1, 0, 4, FAKE) == tq.TQ_ERR_INVALID_ARGUMENT
    assert "positive" in tq.tq_last_error()
    assert tq.tq_codebook_device_bytes(128, 128) == 2 * 128 * 128 * 4 + 2 * 128 * 128 * 2


def test_codebook_init_rejects_before_any_device_call():
    s = tq.tq_codebook_t()
    assert tq._lib.tq_codebook_init(ctypes.byref(s), 64, 3, 1, None, FAKE, None) == tq.TQ_ERR_UNSUPPORTED
    assert tq._lib.tq_codebook_init(ctypes.byref(s), 128, 5, 1, None, FAKE, None) == tq.TQ_ERR_UNSUPPORTED
    assert tq._lib.tq_codebook_init(ctypes.byref(s), 128, 1, 1, None, FAKE, None) == tq.TQ_ERR_UNSUPPORTED
    assert tq._lib.tq_codebook_init(ctypes.byref(s), 128, 3, 1, None, None, None) == tq.TQ_ERR_INVALID_ARGUMENT
    assert tq._lib.tq_codebook_init(None, 128, 3, 1, None, FAKE, None) == tq.TQ_ERR_INVALID_ARGUMENT
    assert s.magic == 0


def _fake_cb(initialised=True, bits=3):
    s = tq.tq_codebook_t()
    s.head_dim, s.bits, s.qjl_dim, s.block_size = 128, bits, 128, 16
    s.d_tables = FAKE
    s.magic = 0x54513031 if initialised else 0
    return s


def _enc(cb, **kw):
    a = dict(k=FAKE, v=FAKE, dtype=tq.TQ_BF16, T=4, H=2, ts=256, hs=128, slots=FAKE,
             kc=FAKE, vc=FAKE, norms=None)
    a.update(kw)
    return tq._lib.tq_encode_kv(ctypes.byref(cb), a["k"], a["v"], a["dtype"], a["T"], a["H"],
                                a["ts"], a["hs"], a["slots"], a["kc"], a["vc"], a["norms"], None)


def test_encode_validation():
    cb = _fake_cb()
    assert _enc(_fake_cb(False)) == tq.TQ_ERR_NOT_INITIALIZED
    assert tq._lib.tq_encode_kv(None, FAKE, FAKE, 0, 1, 1, 128, 128, FAKE, FAKE, FAKE, None, None) \
        == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, T=-1) == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, H=0) == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, dtype=7) == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, k=None) == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, slots=None) == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, ts=-256) == tq.TQ_ERR_INVALID_ARGUMENT
    assert _enc(cb, ts=64, hs=64) == tq.TQ_ERR_INVALID_ARGUMENT
    assert "overlap" in tq.tq_last_error()
    assert _enc(cb, ts=1028) == tq.TQ_ERR_UNSUPPORTED               # stride not a multiple of 8
    assert _enc(cb, k=FAKE + 2) == tq.TQ_ERR_UNSUPPORTED             # misaligned base
    assert _enc(cb, dtype=tq.TQ_F32, ts=258, hs=128) == tq.TQ_ERR_UNSUPPORTED  # not a multiple of 4
    # zero tokens is a no-op that succeeds without touching anything
    assert _enc(cb, T=0, k=None, v=None, slots=None, kc=None, vc=None) == tq.TQ_OK


def _dec(cb, **kw):
    a = dict(q=FAKE, qd=tq.TQ_BF16, kc=FAKE, vc=FAKE, bt=FAKE, mb=64, cl=FAKE, B=1, q_len=1,
             Hq=32, Hkv=8, maxc=1024, scale=0.0, out=FAKE, od=tq.TQ_F32, tps=0, ws=FAKE,
             wsb=1 << 40)
    a.update(kw)
    return tq._lib.tq_decode_attention(
        ctypes.byref(cb), a["q"], a["qd"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["B"],
        a["q_len"], a["Hq"], a["Hkv"], a["maxc"], a["scale"], a["out"], a["od"], a["tps"],
        a["ws"], a["wsb"], None)


def test_decode_validation():
    cb = _fake_cb()
    E = tq.TQ_ERR_INVALID_ARGUMENT
    assert _dec(_fake_cb(False)) == tq.TQ_ERR_NOT_INITIALIZED
    assert _dec(cb, q=None) == E
    assert _dec(cb, ws=None) == E
    assert _dec(cb, qd=9) == E
    assert _dec(cb, od=-1) == E
    assert _dec(cb, B=0) == E
    assert _dec(cb, q_len=0) == E
    assert _dec(cb, Hq=30, Hkv=8) == E
    assert "multiple" in tq.tq_last_error()
    assert _dec(cb, Hq=64, Hkv=2) == tq.TQ_ERR_UNSUPPORTED      # 32 heads per KV head
    assert _dec(cb, Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED      # 17 heads per KV head
    assert _dec(cb, maxc=-1) == E
    assert _dec(cb, q_len=8, maxc=4, mb=1) == E                  # more queries than context
    assert _dec(cb, mb=63) == E                                  # 63 blocks < 1024 tokens
    assert _dec(cb, tps=100) == E
    assert _dec(cb, tps=-256) == E
    assert _dec(cb, scale=float("nan")) == E
    assert _dec(cb, scale=-1.0) == E
    need = tq._lib.tq_decode_workspace_bytes(ctypes.byref(cb), 1, 1, 32, 8, 1024, 0)
    assert need > 0
    assert _dec(cb, wsb=need - 1) == tq.TQ_ERR_WORKSPACE_TOO_SMALL
    # a verify block of 16 query rows per KV head (4 positions x 4 heads) keeps
    # its query operands in the workspace: it must be 16-byte aligned
    assert _dec(cb, q_len=4, ws=FAKE + 8) == E
    assert "aligned" in tq.tq_last_error()


def _prep_words(B, q_len, Hq, Hkv):
    """Query prep floats: the vector and prefill passes keep q' and s (256
    floats) per query row; the matrix-core decode pass (up to 8 heads per KV
    head, at most 4 launches of 8 // G positions) forms its operands inside
    the split pass and keeps none."""
    G = Hq // Hkv
    if G <= 8 and -(-q_len // (8 // G)) <= 4:
        return 0
    return B * q_len * Hq * 256


def _balanced_records(lengths, Hkv, per_fixed, target, min_tiles=4):
    """Records per group under the balanced plan of the matrix-core pass, by
    brute force: tiles of 128 tokens; each (sequence, KV head) group cut into
    ranges of per tiles, per fixed or the smallest multiple of 4 in
    [min_tiles, 64] whose ranges over all groups number at most ``target``
    (else 64)."""
    T = [(int(L) + 127) // 128 for L in lengths]

    def ranges(p):
        return Hkv * sum(-(-t // p) for t in T)
    per = per_fixed or next((p for p in range(min_tiles, 65, 4) if ranges(p) <= target), 64)
    return [-(-t // per) for t in T for _ in range(Hkv)], per


@pytest.mark.parametrize("B,q_len,Hq,Hkv", [(1, 1, 32, 8), (2, 1, 32, 4), (1, 1, 32, 32),
                                            (1, 4, 32, 8), (16, 1, 32, 8), (2, 2, 32, 8)])
def test_workspace_plan_covers_every_record(B, q_len, Hq, Hkv):
    cb = _fake_cb()
    ref = ctypes.byref(cb)
    rows = B * q_len * Hq
    G = Hq // Hkv
    rng = np.random.default_rng(B * 100 + Hkv)
    for maxc, tps in ((8192, 256), (8192, 1024), (131072, 0), (32768, 0), (0, 0), (1, 0)):
        maxc = max(maxc, q_len)
        if q_len > 1 and G * q_len > 8 and tps == 0:
            continue  # the stream plan (test_stream_plan_covers_every_tile_within_the_workspace)
        ws = tq._lib.tq_decode_workspace_bytes(ref, B, q_len, Hq, Hkv, maxc, tps)
        words = ws // 4 - _prep_words(B, q_len, Hq, Hkv)
        assert ws % 4 == 0 and words % (rows * 132) == 0
        recs = words // (rows * 132)
        assert recs >= 1
        # the ranges should fill the 256 compute units once: 8-wave
        # workgroups for 5 to 8 query rows, two 4-wave ones per unit for up to 4
        mrows = G * min(q_len, 8 // G)
        target = 256 if mrows > 4 else 512
        for trial in range(20):
            if trial == 0:
                lengths = np.full(B, maxc)
            else:
                lengths = np.minimum(np.floor(np.exp(rng.uniform(0, np.log(maxc + 1), B))), maxc)
                lengths[rng.integers(B)] = maxc
            counts, per = _balanced_records(lengths, Hkv, tps // 128, target)
            assert per <= 64
            assert max(counts, default=0) <= recs, (maxc, tps, trial, max(counts), recs)
    assert tq._lib.tq_decode_workspace_bytes(ref, 0, 1, 32, 8, 10, 0) == 0
    assert tq._lib.tq_k_page_bytes(ref) == 1088 and tq._lib.tq_v_page_bytes(ref) == 800


def test_workspace_of_the_vector_and_prefill_passes():
    # chunks of tokens_per_split per (sequence or query block, KV head)
    cb = _fake_cb()
    ref = ctypes.byref(cb)
    for B, q_len, Hq, Hkv in ((1, 1, 32, 2), (2, 21, 32, 8)):
        rows = B * q_len * Hq
        for maxc, tps in ((8192, 256), (8192, 1024)):
            ws = tq._lib.tq_decode_workspace_bytes(ref, B, q_len, Hq, Hkv, maxc, tps)
            words = ws // 4 - _prep_words(B, q_len, Hq, Hkv)
            assert words == rows * 132 * max(1, -(-maxc // tps))


def _hot(cb, **kw):
    a = dict(q=FAKE, qd=tq.TQ_BF16, kc=FAKE, vc=FAKE, bt=FAKE, mb=64, cl=FAKE, B=1,
             Hq=32, Hkv=8, maxc=1024, hk=FAKE, hv=FAKE, hd=tq.TQ_BF16, hl=FAKE, hmax=300,
             scale=0.0, out=FAKE, od=tq.TQ_F32, tps=0, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return tq._lib.tq_decode_attention_hot(
        ctypes.byref(cb), a["q"], a["qd"], a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["B"],
        a["Hq"], a["Hkv"], a["maxc"], a["hk"], a["hv"], a["hd"], a["hl"], a["hmax"], a["scale"],
        a["out"], a["od"], a["tps"], a["ws"], a["wsb"], None)


def test_hot_window_validation():
    cb = _fake_cb()
    E = tq.TQ_ERR_INVALID_ARGUMENT
    assert _hot(_fake_cb(False)) == tq.TQ_ERR_NOT_INITIALIZED
    assert _hot(cb, q=None) == E                                  # the plain call's checks
    assert _hot(cb, Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED       # 17 heads per KV head
    assert _hot(cb, hmax=-1) == E
    assert _hot(cb, hk=None) == E
    assert _hot(cb, hl=None) == E
    assert _hot(cb, hd=7) == E
    assert _hot(cb, hv=FAKE + 8) == tq.TQ_ERR_UNSUPPORTED         # misaligned window
    ref = ctypes.byref(cb)
    need = tq._lib.tq_decode_hot_workspace_bytes(ref, 1, 32, 8, 1024, 300, 0)
    assert _hot(cb, wsb=need - 1) == tq.TQ_ERR_WORKSPACE_TOO_SMALL
    # no window: the plain decode workspace; a window of 300 tokens adds five
    # partial records (64-token chunks) per query row
    plain = tq._lib.tq_decode_workspace_bytes(ref, 1, 1, 32, 8, 1024, 0)
    assert tq._lib.tq_decode_hot_workspace_bytes(ref, 1, 32, 8, 1024, 0, 0) == plain
    assert need == plain + 32 * 5 * 132 * 4
    assert tq._lib.tq_decode_hot_workspace_bytes(ref, 1, 32, 8, 1024, -1, 0) == 0


def test_oversized_chunk_is_rejected_not_clamped():
    # the matrix-core decode pass takes at most 8,192 tokens per chunk; an
    # explicit larger request is an error (the automatic plan stays below)
    cb = _fake_cb()
    assert _dec(cb, maxc=32768, mb=2048, tps=8192 + 256) == tq.TQ_ERR_UNSUPPORTED
    assert "exceeds" in tq.tq_last_error()
    # (an accepted 8,192-token request would launch: that case runs in the GPU tests)
    ref = ctypes.byref(cb)
    # automatic plan for many (sequence, KV head) groups of up to 131,072
    # tokens: ranges found on the device fill 512 workgroups, so a group
    # spans at most 512 / 8 of them
    ws = tq._lib.tq_decode_workspace_bytes(ref, 128, 1, 32, 8, 131072, 0)
    assert ws // 4 == 128 * 32 * 64 * 132


def test_binding_rejects_mismatched_pools_before_any_launch():
    # the pools reach the C ABI as bare pointers, so the binding checks their
    # dtype, layout and page sizes; these all fail before any device call
    import torch
    cb = tq.Codebook(_fake_cb(), None)
    q = torch.zeros((1, 1, 32, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    cl = torch.zeros(1, dtype=torch.int32)
    good_k = torch.zeros((4, 8, 1088), dtype=torch.uint8)
    good_v = torch.zeros((4, 8, 800), dtype=torch.uint8)
    bad = [
        (torch.zeros((4, 4, 1088), dtype=torch.uint8), good_v, "k_cache"),    # other head count
        (good_k, torch.zeros((4, 8, 1088), dtype=torch.uint8), "v_cache"),    # K page size for V
        (good_k.to(torch.int16), good_v, "uint8"),
        (good_k, good_v[:, :, :400], "v_cache"),
        (good_k, torch.zeros((5, 8, 800), dtype=torch.uint8), "same number"),
        (good_k.transpose(0, 1), good_v, "contiguous"),
    ]
    for kc, vc, msg in bad:
        with pytest.raises((ValueError, TypeError), match=msg):
            tq.tq_decode_attention(cb, q, kc, vc, bt, cl, 64, 8)
    with pytest.raises(ValueError, match="block_tables"):
        tq.tq_decode_attention(cb, q, good_k, good_v, torch.zeros((2, 4), dtype=torch.int32), cl, 64, 8)
    with pytest.raises(ValueError, match="context_lens"):
        tq.tq_decode_attention(cb, q, good_k, good_v, bt, torch.zeros(3, dtype=torch.int32), 64, 8)
    hk = torch.zeros((1, 16, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="hot_lens"):
        tq.tq_decode_attention_hot(cb, q, good_k, good_v, bt, cl, 64, 8, hk, hk,
                                   torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="k_cache"):
        tq.tq_decode_attention_hot(cb, q, good_k[:, :4].contiguous(), good_v, bt, cl, 64, 8, hk, hk,
                                   torch.zeros(1, dtype=torch.int32))
    k = torch.zeros((16, 8, 128), dtype=torch.bfloat16)
    slots = torch.zeros(16, dtype=torch.int64)
    with pytest.raises(ValueError, match="k_cache"):
        tq.tq_encode_kv(cb, k, k, slots, torch.zeros((4, 2, 1088), dtype=torch.uint8), good_v)
    with pytest.raises(ValueError, match="slot_mapping"):
        tq.tq_encode_kv(cb, k, k, slots[:8], good_k, good_v)
    with pytest.raises(ValueError, match="norms_out"):
        tq.tq_encode_kv(cb, k, k, slots, good_k, good_v, norms_out=torch.zeros((16, 8, 2)))


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_device_call():
    cb = _fake_cb()
    ref = ctypes.byref(cb)
    cap = tq.tq_decode_noalloc_scratch_bytes()
    assert cap == 64 << 20

    def call(**kw):
        a = dict(B=1, q_len=1, Hq=32, Hkv=8, maxc=1024, mb=64)
        a.update(kw)
        return tq._lib.tq_decode_attention_noalloc(
            ref, FAKE, tq.TQ_BF16, FAKE, FAKE, FAKE, a["mb"], FAKE, a["B"], a["q_len"], a["Hq"],
            a["Hkv"], a["maxc"], 0.0, FAKE, tq.TQ_F32, 0, None)
    # 256 sequences x 32 heads over 131,072 tokens: 64 partial records per row
    need = tq._lib.tq_decode_workspace_bytes(ref, 256, 1, 32, 8, 131072, 0)
    assert need > cap
    assert call(B=256, maxc=131072, mb=8192) == tq.TQ_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in tq.tq_last_error()
    # the plain call's argument checks come first
    assert call(Hq=30) == tq.TQ_ERR_INVALID_ARGUMENT
    assert tq._lib.tq_decode_attention_noalloc(
        ctypes.byref(_fake_cb(False)), FAKE, tq.TQ_BF16, FAKE, FAKE, FAKE, 64, FAKE, 1, 1, 32, 8, 1024,
        0.0, FAKE, tq.TQ_F32, 0, None) == tq.TQ_ERR_NOT_INITIALIZED
    assert tq._lib.tq_decode_attention_noalloc(
        ref, None, tq.TQ_BF16, FAKE, FAKE, FAKE, 64, FAKE, 1, 1, 32, 8, 1024,
        0.0, FAKE, tq.TQ_F32, 0, None) == tq.TQ_ERR_INVALID_ARGUMENT


def _win(cb, **kw):
    a = dict(q=FAKE, qd=tq.TQ_BF16, kc=FAKE, vc=FAKE, bt=FAKE, rb=70, cl=FAKE, B=1, q_len=1,
             Hq=32, Hkv=8, maxc=100000, W=1024, scale=0.0, out=FAKE, od=tq.TQ_F32, tps=0, ws=FAKE,
             wsb=1 << 40)
    a.update(kw)
    return tq._lib.tq_decode_attention_window(
        ctypes.byref(cb), a["q"], a["qd"], a["kc"], a["vc"], a["bt"], a["rb"], a["cl"], a["B"],
        a["q_len"], a["Hq"], a["Hkv"], a["maxc"], a["W"], a["scale"], a["out"], a["od"], a["tps"],
        a["ws"], a["wsb"], None)


def test_window_validation():
    """Checks of the sliding-window call that run before any launch: the
    window, the ring size against window + q_len - 1, the plain call's
    checks, and the workspace (every case below fails on the host)."""
    cb = _fake_cb()
    E = tq.TQ_ERR_INVALID_ARGUMENT
    assert _win(_fake_cb(False)) == tq.TQ_ERR_NOT_INITIALIZED
    assert _win(cb, W=0) == E
    assert "window" in tq.tq_last_error()
    assert _win(cb, W=-5) == E
    assert _win(cb, rb=63) == E                      # 63 pages < 1024 positions
    assert "ring" in tq.tq_last_error()
    assert _win(cb, rb=64, q_len=2) == E             # 1025 positions needed
    assert _win(cb, q=None) == E
    assert _win(cb, Hq=30) == E
    assert _win(cb, Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED
    assert _win(cb, wsb=16) == tq.TQ_ERR_WORKSPACE_TOO_SMALL
    assert _win(cb, ws=None) == E


def test_window_workspace_covers_only_the_window():
    """The window call plans over about window + q_len - 1 + 15 positions per
    sequence whatever the context length; a window covering the context
    plans exactly like the plain call."""
    cb = ctypes.byref(_fake_cb())
    plain_fn, win_fn = tq._lib.tq_decode_workspace_bytes, tq._lib.tq_decode_window_workspace_bytes
    plain = plain_fn(cb, 16, 1, 32, 8, 131072, 0)
    win = win_fn(cb, 16, 1, 32, 8, 131072, 1024, 0)
    assert 0 < win < plain
    assert win == win_fn(cb, 16, 1, 32, 8, 2 ** 30, 1024, 0)
    for q_len, Hq, Hkv in [(1, 32, 8), (3, 32, 4), (21, 16, 2), (1, 32, 2)]:
        assert win_fn(cb, 4, q_len, Hq, Hkv, 5000, 5000, 0) == plain_fn(cb, 4, q_len, Hq, Hkv, 5000, 0)
    assert win_fn(cb, 4, 1, 32, 8, 5000, 0, 0) == 0


def test_page_sizes_and_plans_of_the_other_bit_widths():
    """2 and 4-bit codebooks: page sizes 256 (b + 1) + 64 and 256 b + 32, as
    the oracle's layout, and a decode plan on the vector pass (query
    operands in the workspace) where 3 bits take the matrix-core pass."""
    from oracle import pages as P
    for b in (2, 3, 4):
        cb = ctypes.byref(_fake_cb(bits=b))
        assert tq._lib.tq_k_page_bytes(cb) == P.k_page_bytes(b)
        assert tq._lib.tq_v_page_bytes(cb) == P.v_page_bytes(b)
    w3 = tq._lib.tq_decode_workspace_bytes(ctypes.byref(_fake_cb(bits=3)), 4, 1, 32, 8, 8192, 0)
    for b in (2, 4):
        wb = tq._lib.tq_decode_workspace_bytes(ctypes.byref(_fake_cb(bits=b)), 4, 1, 32, 8, 8192, 0)
        assert wb > w3 and wb >= 4 * 32 * 256 * 4      # query operands of every row come first



def _step(cb, **kw):
    a = dict(k=FAKE, v=FAKE, kd=tq.TQ_BF16, ts=1024, hs=128, slots=FAKE, q=FAKE, qd=tq.TQ_BF16,
             kc=FAKE, vc=FAKE, bt=FAKE, mb=64, cl=FAKE, B=2, Hq=32, Hkv=8, maxc=1024, scale=0.0,
             out=FAKE, od=tq.TQ_F32, tps=0, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return tq._lib.tq_decode_step(
        ctypes.byref(cb), a["k"], a["v"], a["kd"], a["ts"], a["hs"], a["slots"], a["q"], a["qd"],
        a["kc"], a["vc"], a["bt"], a["mb"], a["cl"], a["B"], a["Hq"], a["Hkv"], a["maxc"], a["scale"],
        a["out"], a["od"], a["tps"], a["ws"], a["wsb"], None)


def test_step_validation():
    """Checks of the fused decode step that run before any launch: those of
    the append (its new tokens, strides, alignment), those of the attention
    call, and the workspace's size and alignment (every case fails on the
    host, so nothing is launched)."""
    cb = _fake_cb()
    E = tq.TQ_ERR_INVALID_ARGUMENT
    assert _step(_fake_cb(False)) == tq.TQ_ERR_NOT_INITIALIZED
    assert _step(cb, B=0) == E
    assert _step(cb, k=None) == E
    assert _step(cb, slots=None) == E
    assert _step(cb, kd=7) == E
    assert _step(cb, ts=64, hs=64) == E
    assert "overlap" in tq.tq_last_error()
    assert _step(cb, k=FAKE + 2) == tq.TQ_ERR_UNSUPPORTED
    assert _step(cb, ws=FAKE + 8) == E
    assert "aligned" in tq.tq_last_error()
    assert _step(cb, q=None) == E
    assert _step(cb, Hq=30) == E
    assert _step(cb, Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED
    assert _step(cb, mb=63) == E
    assert _step(cb, scale=float("nan")) == E
    need = tq._lib.tq_decode_step_workspace_bytes(ctypes.byref(cb), 2, 32, 8, 1024, 0)
    assert _step(cb, wsb=need - 1) == tq.TQ_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("bits,Hq,Hkv,fused", [(3, 32, 8, True), (3, 8, 8, True), (3, 16, 8, True),
                                                (3, 64, 8, True), (3, 40, 8, True), (3, 72, 8, False),
                                                (2, 32, 8, False), (4, 32, 8, False)])
def test_step_workspace(bits, Hq, Hkv, fused):
    """The fused step's split pass runs the stream plan: 16 sequences of up
    to 32,768 tokens x Hkv KV heads are at most 16 x Hkv x 256 tiles, so at
    most max(2,048, tiles / 16) runs of tiles; it needs one record (132
    floats) per query head of the group at each of runs + groups places, then
    the query operands (44 words per lane of a 64-lane wave) of each
    (sequence, KV head) group and head tile (two tiles for 5 to 8 heads),
    then a descriptor of 256 words per wave of the split pass's grid and two
    words per group for the merge.  An unfused step needs the attention
    call's workspace."""
    cb = ctypes.byref(_fake_cb(bits=bits))
    B, ctx = 16, 32768
    dec = tq._lib.tq_decode_workspace_bytes(cb, B, 1, Hq, Hkv, ctx, 0)
    step = tq._lib.tq_decode_step_workspace_bytes(cb, B, Hq, Hkv, ctx, 0)
    if fused:
        G = Hq // Hkv
        runs = max(2048, -(-(B * Hkv * 256) // 16))
        P = 2 if G > 4 else 1
        grid = (P * runs + 3) // 4 + 7
        assert step == ((runs + B * Hkv) * G * 132 * 4 + B * Hkv * P * 44 * 64 * 4 + grid * 4 * 256 * 4
                        + B * Hkv * 8)
    else:
        assert step == dec


def _stream_plan(lengths, Hkv, rows, target=512):
    """The stream plan as the split pass and the merge compute it (a restatement
    on the host of their index arithmetic) for groups of `rows` query rows
    (G q_len): tile counts, runs, waves per run and the groups' starts."""
    T = [(int(L) + 127) // 128 for L in lengths]
    N = Hkv * sum(T)
    P = -(-rows // 4)
    q = min(max(-(-(P * N) // (4 * target)), 1), 16)
    runs = -(-N // q)
    nwg = (P * runs + 3) // 4
    # the groups' first tiles in the order (sequence-major, then KV head)
    starts, g = {}, 0
    c = 0
    for b, t in enumerate(T):
        for h in range(Hkv):
            starts[b * Hkv + h] = (c, t)
            c += t
    owner = []  # global tile -> group
    for grp in range(len(T) * Hkv):
        owner += [grp] * starts[grp][1]
    return dict(N=N, P=P, q=q, runs=runs, nwg=nwg, starts=starts, owner=owner)


def _xcd_run_start(x, total):
    return (x * total + 7) // 8


@pytest.mark.parametrize("G,q_len", [(1, 1), (3, 1), (4, 1), (5, 1), (8, 1), (4, 3), (4, 8), (8, 2), (8, 4),
                                     (3, 8), (1, 32), (6, 4)])
def test_stream_plan_covers_every_tile_within_the_workspace(G, q_len):
    """CPU restatement of the stream plan's indexing (the fused decode step,
    q_len 1, and verify blocks of more than 8 query rows per KV head),
    checked against the workspace the library sizes: over ragged batches,
    single long sequences and empty ones, every (tile, head tile) is taken by
    exactly one wave, every record place and row lies inside the records,
    every operand item inside the operands, the grid reaches every workgroup
    of the plan, and the merge reads exactly the places the split pass
    writes."""
    cb = ctypes.byref(_fake_cb())
    rng = np.random.default_rng(100 + G + 7 * q_len)
    rows = G * q_len
    cases = [([131072], 4), ([1], 8), ([0, 0, 5], 2), ([32768] * 16, 8), ([100000, 131072], 8), ([16] * 64, 8),
             (list(range(0, 4000, 37)), 2)]
    for _ in range(12):
        B = int(rng.integers(1, 40))
        hi = int(rng.choice([600, 4096, 40000]))
        cases.append((list(rng.integers(0, hi, B)), int(rng.choice([1, 2, 4, 8]))))
    for lengths, Hkv in cases:
        B, maxc = len(lengths), max(max(lengths), q_len)
        Hq = G * Hkv
        plan = _stream_plan(lengths, Hkv, rows)
        N, P, q, runs, nwg = plan["N"], plan["P"], plan["q"], plan["runs"], plan["nwg"]
        groups = B * Hkv
        # the host's bound on runs, places and the grid
        run_bound = max(2048, -(-(B * Hkv * ((maxc + 127) // 128)) // 16))
        grid = (P * run_bound + 3) // 4 + 7
        if q_len == 1:
            ws = tq._lib.tq_decode_step_workspace_bytes(cb, B, Hq, Hkv, maxc, 0)
        else:
            ws = tq._lib.tq_decode_workspace_bytes(cb, B, q_len, Hq, Hkv, maxc, 0)
        assert ws == ((run_bound + groups) * rows * 132 * 4 + groups * P * 44 * 64 * 4 + grid * 4 * 256 * 4
                      + groups * 8)
        assert runs <= run_bound
        # workgroups: blockIdx -> (die x, place in the die's run)
        reached = set()
        for blk in range(grid):
            x, s = blk & 7, blk >> 3
            rpos = _xcd_run_start(x, nwg) + s
            if rpos < _xcd_run_start(x + 1, nwg):
                assert rpos not in reached
                reached.add(rpos)
        assert reached == set(range(nwg))
        covered = {}
        written = {}
        items = set()
        for rpos in range(nwg):
            for wave in range(4):
                iw, ut = divmod(4 * rpos + wave, P)
                ntiles = min(q, N - iw * q)
                if ntiles <= 0:
                    continue
                touched = set()
                for k in range(ntiles):
                    c = iw * q + k
                    grp = plan["owner"][c]
                    key = (c, ut)
                    assert key not in covered
                    covered[key] = True
                    touched.add(grp)
                for grp in touched:
                    items.add(grp * P + ut)
                    for row in range(4 * ut, min(4 * ut + 4, rows)):
                        place = iw + grp
                        assert place < run_bound + groups
                        written.setdefault(grp, set()).add((place, row))
        assert set(covered) == {(c, u) for c in range(N) for u in range(P)}
        assert items <= set(range(groups * P))
        # the merge: group g's records are places floor(C/q) + g .. floor((C + T - 1)/q) + g
        for grp, (c0, t) in plan["starts"].items():
            if t == 0:
                assert grp not in written
                continue
            places = set(range(c0 // q + grp, (c0 + t - 1) // q + grp + 1))
            assert written[grp] == {(p, r) for p in places for r in range(rows)}
