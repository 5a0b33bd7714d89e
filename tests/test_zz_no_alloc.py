"""The no-allocation decode entry point against the plain one (same kernels,
same chunk plan): two calls in a row on the library's device scratch, the
second with a smaller input, each equal to tq_decode_attention's output."""
import numpy as np
import pytest
import torch

import synth
import decode_attention_tq_amd as tq
from gpu_helpers import codebook, dev, encode_gpu, new_pools

pytestmark = pytest.mark.gpu


def _case(seed, lens, Hq, Hkv, q_len=1):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    table, nb = synth.block_tables(rng, lens)
    cb = codebook()
    kpool, vpool = new_pools(nb, Hkv)
    for b in range(len(lens)):
        k = synth.kv_tensor(rng, int(lens[b]), Hkv)
        v = synth.kv_tensor(rng, int(lens[b]), Hkv)
        encode_gpu(cb, k, v, synth.slots_for(table, b, np.arange(lens[b])), kpool, vpool, with_norms=False)
    q = dev(synth.queries(rng, len(lens), q_len, Hq), torch.bfloat16)
    return cb, q, kpool, vpool, torch.from_numpy(table).cuda(), torch.from_numpy(lens.astype(np.int32)).cuda(), \
        int(lens.max())


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    big = _case(50, [3000, 9000, 700, 12000], 32, 8)
    small = _case(51, [500, 1300], 32, 4)
    for cb, q, kp, vp, bt, cl, maxc in (big, small):
        Hkv = kp.shape[1]
        ref = tq.tq_decode_attention(cb, q, kp, vp, bt, cl, maxc, Hkv)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_decode_attention_noalloc(cb, q, kp, vp, bt, cl, maxc, Hkv, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), float((out - ref).abs().max())


def test_noalloc_verify_block_on_the_stream_plan():
    """A verify block of 16 query rows per KV head (4 positions x 4 heads)
    keeps its query operands and partial records in the device scratch: two
    calls in a row, the second smaller, each equal to the workspace call."""
    big = _case(52, [3000, 9000, 700], 32, 8, q_len=4)
    small = _case(53, [500, 1300], 16, 2, q_len=3)
    for cb, q, kp, vp, bt, cl, maxc in (big, small):
        Hkv = kp.shape[1]
        ref = tq.tq_decode_attention(cb, q, kp, vp, bt, cl, maxc, Hkv)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_decode_attention_noalloc(cb, q, kp, vp, bt, cl, maxc, Hkv, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), float((out - ref).abs().max())
