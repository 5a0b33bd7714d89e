"""2- and 4-bit codebook variants through the HIP path (C ABI) against the
oracle: encode bit-exact outside the threshold band (bf16 and fp32 inputs,
whole pages and token-by-token appends into partial pages), then decode over
the pages (the vector pass serves these widths) for single-query decode, a
verify block and a sliding window, 4 and 16 heads per KV head."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (check_decode, check_encoded_sequence, codebook, decode_gpu, dev, encode_gpu, new_pools,
                         oracle_tables, assert_rows_close)
from oracle import decode_paged_window
import decode_attention_tq_amd as tq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float32])
def test_encode_bit_exact_at_other_widths(bits, in_dtype):
    T, Hkv = 1003, 8
    case = synth.gqa_case(seed=80 + bits, T=T, Hq=32, Hkv=Hkv)
    cb = codebook(bits=bits)
    assert tq.tq_k_page_bytes(cb) == 256 * (bits + 1) + 64 and tq.tq_v_page_bytes(cb) == 256 * bits + 32
    kpool, vpool = new_pools(case["num_blocks"], Hkv, bits=bits)
    n0 = T - 5
    norms = encode_gpu(cb, case["k"][:n0], case["v"][:n0], case["slots"][:n0], kpool, vpool, dtype=in_dtype)
    tail = []
    for j in range(n0, T):  # one token per call into the partly filled last pages
        tail.append(encode_gpu(cb, case["k"][j:j + 1], case["v"][j:j + 1], case["slots"][j:j + 1], kpool, vpool,
                               dtype=in_dtype))
    norms = np.concatenate([norms] + tail)
    k = case["k"] if in_dtype == torch.bfloat16 else case["k"].astype(np.float32)
    v = case["v"] if in_dtype == torch.bfloat16 else case["v"].astype(np.float32)
    stats = {}
    check_encoded_sequence(k, v, kpool.cpu().numpy(), vpool.cpu().numpy(), case["table"][0], np.arange(T), norms,
                           tables=oracle_tables(bits=bits), stats=stats)
    print("bits", bits, stats)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 2)])
def test_decode_at_other_widths(bits, Hq, Hkv):
    rng = np.random.default_rng(90 + bits)
    lens = np.array([700, 2300, 37], dtype=np.int64)
    table, nb = synth.block_tables(rng, lens)
    cb = codebook(bits=bits)
    kpool, vpool = new_pools(nb, Hkv, bits=bits)
    for b in range(len(lens)):
        k = synth.kv_tensor(rng, int(lens[b]), Hkv)
        v = synth.kv_tensor(rng, int(lens[b]), Hkv)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    kp, vp = kpool.cpu().numpy(), vpool.cpu().numpy()
    tables = oracle_tables(bits=bits)
    cl = lens.astype(np.int32)
    for q_len in (1, 3):
        q = synth.queries(rng, len(lens), q_len, Hq)
        out = decode_gpu(cb, q, kpool, vpool, table, cl, Hkv)
        err = check_decode(out, q, kp, vp, table, cl, tables=tables)
        print("bits", bits, "G", Hq // Hkv, "q_len", q_len, "max rel err", err.max())
    # a sliding window over the same (linear) table
    q = synth.queries(rng, len(lens), 1, Hq)
    out = tq.tq_decode_attention_window(cb, dev(q, torch.bfloat16), kpool, vpool, torch.from_numpy(table).cuda(),
                                        torch.from_numpy(cl).cuda(), int(lens.max()), Hkv, 300)
    torch.cuda.synchronize()
    c32, _, S = tables
    ref = decode_paged_window(q, kp, vp, table, lens, 300, c32, S)
    assert_rows_close(out.float().cpu().numpy(), ref)
