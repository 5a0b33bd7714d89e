"""Sliding-window decode over a rotating compressed cache (HIP path through
the C ABI) against the oracle: the ring of pages holds only the positions
the windows can reach, older pages are overwritten, and every pass (the
matrix-core pass for up to 8 heads per KV head, the vector pass, the prefill
pass for a long query block) sees only its window."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_rows_close, codebook, dev, encode_gpu, new_pools, oracle_tables
from oracle import decode_paged_window
import decode_attention_tq_amd as tq

pytestmark = pytest.mark.gpu


def _ring_pools(rng, lens, Hkv, R, chunk=256):
    """Every sequence's tokens written in position order into its ring of R
    pages, ``chunk`` positions per encode call (older positions overwritten)."""
    B = len(lens)
    nb = B * R + 5
    table = rng.permutation(nb)[:B * R].reshape(B, R).astype(np.int32)
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv, seed=int(rng.integers(1 << 30)))
    for b, L in enumerate(lens):
        k = synth.kv_tensor(rng, int(L), Hkv)
        v = synth.kv_tensor(rng, int(L), Hkv)
        for s in range(0, int(L), chunk):
            j = np.arange(s, min(s + chunk, int(L)))
            slots = table[b][(j // 16) % R].astype(np.int64) * 16 + j % 16
            encode_gpu(cb, k[j], v[j], slots, kpool, vpool, with_norms=False)
    return cb, table, kpool, vpool


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 4), (32, 2), (12, 4)])
def test_sliding_window_over_a_ring(Hq, Hkv):
    rng = np.random.default_rng(70 + Hq // Hkv)
    W, R = 500, 36                               # 576 ring positions >= W + 21 - 1
    lens = np.array([25, 700, 3001, 517], dtype=np.int64)
    cb, table, kpool, vpool = _ring_pools(rng, lens, Hkv, R)
    kp, vp = kpool.cpu().numpy(), vpool.cpu().numpy()
    c32, _, S = oracle_tables()
    bt = torch.from_numpy(table).cuda()
    cl = torch.from_numpy(lens.astype(np.int32)).cuda()
    for q_len, tps in ((1, 0), (3, 0), (21, 0), (21, 256), (1, 256)):
        q = synth.queries(rng, len(lens), q_len, Hq)
        out = tq.tq_decode_attention_window(cb, dev(q, torch.bfloat16), kpool, vpool, bt, cl, int(lens.max()),
                                            Hkv, W, tokens_per_split=tps)
        torch.cuda.synchronize()
        ref = decode_paged_window(q, kp, vp, table, lens, W, c32, S)
        err = assert_rows_close(out.float().cpu().numpy(), ref)
        print("G", Hq // Hkv, "q_len", q_len, "tps", tps, "max rel err", err.max())


def test_window_covering_the_context_is_the_plain_call():
    """A window as long as the context over a table that never wraps plans
    and computes exactly like tq_decode_attention: bit-identical output."""
    rng = np.random.default_rng(77)
    lens = np.array([700, 2300], dtype=np.int64)
    table, nb = synth.block_tables(rng, lens)
    cb = codebook()
    kpool, vpool = new_pools(nb, 8)
    for b in range(len(lens)):
        k = synth.kv_tensor(rng, int(lens[b]), 8)
        v = synth.kv_tensor(rng, int(lens[b]), 8)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    q = dev(synth.queries(rng, 2, 1, 32), torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    cl = torch.from_numpy(lens.astype(np.int32)).cuda()
    plain = tq.tq_decode_attention(cb, q, kpool, vpool, bt, cl, 2300, 8)
    win = tq.tq_decode_attention_window(cb, q, kpool, vpool, bt, cl, 2300, 8, 2300)
    torch.cuda.synchronize()
    assert torch.equal(plain, win)
