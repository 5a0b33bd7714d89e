"""Pins of the page layout: sizes, bit positions, round trips, fast forms."""
import numpy as np
import pytest

from oracle import pages as P


def test_page_sizes_give_the_pages_bit_widths():
    assert P.K_PAGE_BYTES == 1088 and P.V_PAGE_BYTES == 800
    assert P.K_PAGE_BYTES * 8 / (P.BLOCK * P.HEAD_DIM) == 4.25
    assert P.V_PAGE_BYTES * 8 / (P.BLOCK * P.HEAD_DIM) == 3.125
    overall = (P.K_PAGE_BYTES + P.V_PAGE_BYTES) * 8 / (2 * P.BLOCK * P.HEAD_DIM)
    assert overall == 3.6875
    assert abs(16 / overall - 4.339) < 1e-3


def test_hand_placed_bits():
    codes = np.zeros((16, 128), np.uint8)
    signs = np.zeros((16, 128), np.uint8)
    codes[3, 9] = 5            # binary 101 -> planes 0 and 2
    signs[3, 9] = 1
    n16 = np.zeros(16, np.float16)
    g16 = np.zeros(16, np.float16)
    n16[3] = np.float16(2.0)   # 0x4000
    g16[3] = np.float16(-0.5)  # 0xB800
    codes[5, 100] = 6          # binary 110 -> planes 1 and 2, chunk 3
    signs[5, 100] = 1
    k = P.pack_k_page(codes, signs, n16, g16)
    # coordinate 9 of token 3: chunk 0, record 16 * (16 * 0 + 3) = 48; field f
    # is the word at 48 + 4 f; bit 9 is byte 1, bit 1 of the word
    assert k[48 + 0 + 1] == 0b10
    assert k[48 + 4 + 1] == 0
    assert k[48 + 8 + 1] == 0b10
    assert k[48 + 12 + 1] == 0b10
    # coordinate 100 of token 5: chunk 3, record 16 * (48 + 5) = 848; bit
    # 100 % 32 = 4 is byte 0, bit 4 of each word
    assert k[848 + 0] == 0
    assert k[848 + 4] == 0b10000
    assert k[848 + 8] == 0b10000
    assert k[848 + 12] == 0b10000
    assert (k[1024 + 6], k[1025 + 6]) == (0x00, 0x40)
    assert (k[1056 + 6], k[1057 + 6]) == (0x00, 0xB8)
    assert int(np.count_nonzero(k)) == 8
    v = P.pack_v_page(codes, n16)
    # coordinate 9's 16-bit word holds token 3 at bit 3
    assert v[0 * 256 + 2 * 9] == 0b1000 and v[0 * 256 + 2 * 9 + 1] == 0
    assert v[2 * 256 + 2 * 9] == 0b1000
    assert v[1 * 256 + 2 * 9] == 0
    # coordinate 100's word holds token 5 at bit 5 (planes 1 and 2)
    assert v[1 * 256 + 2 * 100] == 0b100000 and v[2 * 256 + 2 * 100] == 0b100000
    assert v[0 * 256 + 2 * 100] == 0
    assert (v[768 + 6], v[769 + 6]) == (0x00, 0x40)
    assert int(np.count_nonzero(v)) == 5


def test_round_trips():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 8, (16, 128)).astype(np.uint8)
    signs = rng.integers(0, 2, (16, 128)).astype(np.uint8)
    n16 = rng.uniform(0, 100, 16).astype(np.float16)
    g16 = rng.uniform(0, 1, 16).astype(np.float16)
    c2, s2, n2, g2 = P.unpack_k_page(P.pack_k_page(codes, signs, n16, g16))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, signs)
    np.testing.assert_array_equal(n2, n16)
    np.testing.assert_array_equal(g2, g16)
    c3, n3 = P.unpack_v_page(P.pack_v_page(codes, n16))
    np.testing.assert_array_equal(c3, codes)
    np.testing.assert_array_equal(n3, n16)


def _random_enc(rng, T, H, bits=3):
    return ({"codes": rng.integers(0, 1 << bits, (T, H, 128)).astype(np.uint8),
             "signs": rng.integers(0, 2, (T, H, 128)).astype(np.uint8),
             "norm_f16": rng.uniform(0, 100, (T, H)).astype(np.float16),
             "gamma_f16": rng.uniform(0, 1, (T, H)).astype(np.float16)},
            {"codes": rng.integers(0, 1 << bits, (T, H, 128)).astype(np.uint8),
             "norm_f16": rng.uniform(0, 100, (T, H)).astype(np.float16)})


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fast_writer_and_readers_match_plain_ones(bits):
    rng = np.random.default_rng(1 + bits)
    nb, H, T = 7, 2, 40
    base_k = rng.integers(0, 256, (nb, H, P.k_page_bytes(bits))).astype(np.uint8)
    base_v = rng.integers(0, 256, (nb, H, P.v_page_bytes(bits))).astype(np.uint8)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[[3, 17]] = -1                                   # skipped tokens
    ek, ev = _random_enc(rng, T, H, bits)
    k1, v1 = base_k.copy(), base_v.copy()
    k2, v2 = base_k.copy(), base_v.copy()
    P.write_slots(k1, v1, slots, ek, ev)
    P.write_slots_fast(k2, v2, slots, ek, ev)
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    row = rng.permutation(nb)
    for L in (0, 1, 16, 37, nb * 16):
        for h in range(H):
            a = P.read_k_tokens(k1, row, L, h)
            b = P.read_k_tokens_fast(k1, row, L, h)
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x, y)
            a = P.read_v_tokens(v1, row, L, h)
            b = P.read_v_tokens_fast(v1, row, L, h)
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x, y)


def test_page_sizes_of_the_other_bit_widths():
    """2 and 4-bit codes: one more or one fewer plane per page, same scalars:
    K 3.25 / 5.25 bits and V 2.125 / 4.125 bits per coordinate."""
    assert (P.k_page_bytes(2), P.v_page_bytes(2)) == (832, 544)
    assert (P.k_page_bytes(4), P.v_page_bytes(4)) == (1344, 1056)
    for b, kb, vb in ((2, 3.25, 2.125), (4, 5.25, 4.125)):
        assert P.k_page_bytes(b) * 8 / (P.BLOCK * P.HEAD_DIM) == kb
        assert P.v_page_bytes(b) * 8 / (P.BLOCK * P.HEAD_DIM) == vb
        assert P.k_page_bits(P.k_page_bytes(b)) == b and P.v_page_bits(P.v_page_bytes(b)) == b


def test_hand_placed_bits_at_two_and_four_bits():
    codes = np.zeros((16, 128), np.uint8)
    signs = np.zeros((16, 128), np.uint8)
    n16 = np.zeros(16, np.float16)
    g16 = np.zeros(16, np.float16)
    codes[5, 100] = 2          # binary 10 (or 0010): plane 1
    signs[5, 100] = 1
    n16[5] = np.float16(2.0)   # 0x4000
    g16[5] = np.float16(-0.5)  # 0xB800
    # 2 bits: records of 12 bytes; coordinate 100 of token 5 is chunk 3, record
    # 12 (16 * 3 + 5) = 636, bit 4 of byte 0 of words f = 1 (plane) and 2 (signs)
    k = P.pack_k_page(codes, signs, n16, g16, bits=2)
    assert k[636 + 4] == 0b10000 and k[636 + 8] == 0b10000
    assert (k[768 + 10], k[769 + 10]) == (0x00, 0x40)
    assert (k[800 + 10], k[801 + 10]) == (0x00, 0xB8)
    assert int(np.count_nonzero(k)) == 4
    v = P.pack_v_page(codes, n16, bits=2)
    assert v[256 + 200] == 0b100000 and (v[512 + 10], v[513 + 10]) == (0x00, 0x40)
    assert int(np.count_nonzero(v)) == 2
    # 4 bits: records of 20 bytes; code 9 = 1001 (planes 0 and 3), record
    # 20 (16 * 3 + 5) = 1060, sign in word 4
    codes[5, 100] = 9
    k = P.pack_k_page(codes, signs, n16, g16, bits=4)
    assert k[1060] == 0b10000 and k[1060 + 12] == 0b10000 and k[1060 + 16] == 0b10000
    assert k[1060 + 4] == 0 and k[1060 + 8] == 0
    assert (k[1280 + 10], k[1281 + 10]) == (0x00, 0x40)
    assert (k[1312 + 10], k[1313 + 10]) == (0x00, 0xB8)
    assert int(np.count_nonzero(k)) == 5
    v = P.pack_v_page(codes, n16, bits=4)
    assert v[200] == 0b100000 and v[3 * 256 + 200] == 0b100000
    assert (v[1024 + 10], v[1025 + 10]) == (0x00, 0x40)
    assert int(np.count_nonzero(v)) == 3


@pytest.mark.parametrize("bits", [2, 4])
def test_round_trips_at_other_bit_widths(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, (16, 128)).astype(np.uint8)
    signs = rng.integers(0, 2, (16, 128)).astype(np.uint8)
    n16 = rng.uniform(0, 100, 16).astype(np.float16)
    g16 = rng.uniform(0, 1, 16).astype(np.float16)
    c2, s2, n2, g2 = P.unpack_k_page(P.pack_k_page(codes, signs, n16, g16, bits))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, signs)
    np.testing.assert_array_equal(n2, n16)
    np.testing.assert_array_equal(g2, g16)
    c3, n3 = P.unpack_v_page(P.pack_v_page(codes, n16, bits))
    np.testing.assert_array_equal(c3, codes)
    np.testing.assert_array_equal(n3, n16)

