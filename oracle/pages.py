"""Byte layout of the compressed, paged KV cache (the bit-exact contract).

The pages fix the per-coordinate cost -- 4.25 bits for a key (3-bit code +
1 sign bit + scalars), 3.125 bits for a value ([C] "TurboQuantization", the
K-cache and V-cache headings) -- and that the cache is managed in fixed-size
blocks ([B] "Paged KVキャッシュ").  The byte layout itself is this project's
choice; this module is its independent, plain statement (one bit at a time).

Block = 16 tokens of one KV head, head_dim d = 128, QJL rows m = 128.
Pools: ``k_pool[num_blocks][num_kv_heads][1088]``,
``v_pool[num_blocks][num_kv_heads][800]``; slot = block * 16 + offset.
All multi-byte fields little-endian; bit b of a byte has weight 2^b.

K page (1088 B):
  [0, 1024)     : 64 records of 16 bytes, chunk-major: the record of
      coordinate chunk g = 0..3 (coordinates 32g .. 32g + 31) and token t is
      at 16 (16 g + t); its four little-endian 32-bit words are field
      f = 0, 1, 2 (code bit-plane f: bit i % 32 of the word holds bit f of
      code_i for coordinate i = 32 g + i % 32) and f = 3 (QJL signs: bit
      i % 32 holds the sign bit of projection row i = 32 g + i % 32; 1 means
      z_i >= 0).  So bit f of code_i / the sign of row i sits at byte
      16 (16 (i // 32) + t) + 4 f + (i % 32) // 8, bit i % 8.
  [1024, 1056)  : half n_t at 1024 + 2t.
  [1056, 1088)  : half gamma_t at 1056 + 2t.
V page (800 B):
  [256p, 256p + 256), p = 0, 1, 2 : code bit-plane p, coordinate-major:
      coordinate i owns the 16-bit word at 256p + 2i; its bit t holds bit p
      of token t's code for coordinate i.
  [768, 800)    : half n_t at 768 + 2t.
Bits per coordinate: 1088*8/(16*128) = 4.25 and 800*8/(16*128) = 3.125.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16
HEAD_DIM = 128
QJL_DIM = 128
K_PAGE_BYTES = 3 * 256 + 256 + 2 * BLOCK + 2 * BLOCK
V_PAGE_BYTES = 3 * 256 + 2 * BLOCK


def _put_bit(buf: np.ndarray, byte: int, bit: int, value: int) -> None:
    if value:
        buf[byte] |= np.uint8(1 << bit)
    else:
        buf[byte] &= np.uint8(~(1 << bit) & 0xFF)


def _get_bit(buf: np.ndarray, byte: int, bit: int) -> int:
    return (int(buf[byte]) >> bit) & 1


def _put_half(buf: np.ndarray, off: int, h) -> None:
    raw = np.array([h], dtype=np.float16).view(np.uint16)[0]
    buf[off] = np.uint8(int(raw) & 0xFF)
    buf[off + 1] = np.uint8(int(raw) >> 8)


def _get_half(buf: np.ndarray, off: int) -> np.float16:
    raw = np.uint16(int(buf[off]) | (int(buf[off + 1]) << 8))
    return np.array([raw], dtype=np.uint16).view(np.float16)[0]


def k_bit_byte(t: int, i: int, field: int) -> int:
    """Byte of the K page holding field ``field`` (0..2: code bit-plane,
    3: QJL sign) of coordinate / row ``i`` of token ``t``; the bit is i % 8."""
    return 16 * (16 * (i // 32) + t) + 4 * field + (i % 32) // 8


def set_k_slot(page: np.ndarray, t: int, codes, signs, n16, g16) -> None:
    for i in range(HEAD_DIM):
        for p in range(3):
            _put_bit(page, k_bit_byte(t, i, p), i % 8, (int(codes[i]) >> p) & 1)
    for i in range(QJL_DIM):
        _put_bit(page, k_bit_byte(t, i, 3), i % 8, int(signs[i]))
    _put_half(page, 1024 + 2 * t, n16)
    _put_half(page, 1056 + 2 * t, g16)


def get_k_slot(page: np.ndarray, t: int):
    codes = np.zeros(HEAD_DIM, dtype=np.uint8)
    signs = np.zeros(QJL_DIM, dtype=np.uint8)
    for i in range(HEAD_DIM):
        v = 0
        for p in range(3):
            v |= _get_bit(page, k_bit_byte(t, i, p), i % 8) << p
        codes[i] = v
    for i in range(QJL_DIM):
        signs[i] = _get_bit(page, k_bit_byte(t, i, 3), i % 8)
    return codes, signs, _get_half(page, 1024 + 2 * t), _get_half(page, 1056 + 2 * t)


def set_v_slot(page: np.ndarray, t: int, codes, n16) -> None:
    for i in range(HEAD_DIM):
        for p in range(3):
            word = 256 * p + 2 * i
            _put_bit(page, word + t // 8, t % 8, (int(codes[i]) >> p) & 1)
    _put_half(page, 768 + 2 * t, n16)


def get_v_slot(page: np.ndarray, t: int):
    codes = np.zeros(HEAD_DIM, dtype=np.uint8)
    for i in range(HEAD_DIM):
        v = 0
        for p in range(3):
            v |= _get_bit(page, 256 * p + 2 * i + t // 8, t % 8) << p
        codes[i] = v
    return codes, _get_half(page, 768 + 2 * t)


def pack_k_page(codes, signs, n16, g16) -> np.ndarray:
    """One full K page from ``codes[16][128]``, ``signs[16][128]``, halves."""
    page = np.zeros(K_PAGE_BYTES, dtype=np.uint8)
    for t in range(BLOCK):
        set_k_slot(page, t, codes[t], signs[t], n16[t], g16[t])
    return page


def unpack_k_page(page: np.ndarray):
    out = [get_k_slot(page, t) for t in range(BLOCK)]
    return (np.stack([o[0] for o in out]), np.stack([o[1] for o in out]),
            np.array([o[2] for o in out], dtype=np.float16),
            np.array([o[3] for o in out], dtype=np.float16))


def pack_v_page(codes, n16) -> np.ndarray:
    page = np.zeros(V_PAGE_BYTES, dtype=np.uint8)
    for t in range(BLOCK):
        set_v_slot(page, t, codes[t], n16[t])
    return page


def unpack_v_page(page: np.ndarray):
    out = [get_v_slot(page, t) for t in range(BLOCK)]
    return (np.stack([o[0] for o in out]),
            np.array([o[1] for o in out], dtype=np.float16))


def write_slots(k_pool: np.ndarray, v_pool: np.ndarray, slot_mapping, enc_k: dict,
                enc_v: dict) -> None:
    """Store token ``j``'s records for every KV head at ``slot_mapping[j]``
    (skipped when negative).  ``enc_k``/``enc_v`` hold ``[T][Hkv]`` batches
    from ``encode_k`` / ``encode_v``."""
    T, H = enc_k["codes"].shape[:2]
    for j in range(T):
        s = int(slot_mapping[j])
        if s < 0:
            continue
        blk, off = divmod(s, BLOCK)
        for h in range(H):
            set_k_slot(k_pool[blk, h], off, enc_k["codes"][j, h], enc_k["signs"][j, h],
                       enc_k["norm_f16"][j, h], enc_k["gamma_f16"][j, h])
            set_v_slot(v_pool[blk, h], off, enc_v["codes"][j, h], enc_v["norm_f16"][j, h])


def read_k_tokens(k_pool: np.ndarray, block_row, length: int, head: int):
    """Tokens 0..length-1 of one sequence and KV head, found through its row
    of the block table: (codes[L][128], signs[L][128], n16[L], g16[L])."""
    recs = [get_k_slot(k_pool[int(block_row[j // BLOCK]), head], j % BLOCK)
            for j in range(length)]
    if not recs:
        return (np.zeros((0, HEAD_DIM), np.uint8), np.zeros((0, QJL_DIM), np.uint8),
                np.zeros(0, np.float16), np.zeros(0, np.float16))
    return (np.stack([r[0] for r in recs]), np.stack([r[1] for r in recs]),
            np.array([r[2] for r in recs], dtype=np.float16),
            np.array([r[3] for r in recs], dtype=np.float16))


def read_v_tokens(v_pool: np.ndarray, block_row, length: int, head: int):
    recs = [get_v_slot(v_pool[int(block_row[j // BLOCK]), head], j % BLOCK)
            for j in range(length)]
    if not recs:
        return np.zeros((0, HEAD_DIM), np.uint8), np.zeros(0, np.float16)
    return (np.stack([r[0] for r in recs]),
            np.array([r[1] for r in recs], dtype=np.float16))


# ---------------------------------------------------------------------------
# Vectorised forms of the same layout (np.packbits / np.unpackbits as the
# primitive), for full-size cases.  Pinned against the bit-at-a-time
# functions above by tests/test_oracle_pages.py.

def _pack_bits_le(bits: np.ndarray) -> np.ndarray:
    return np.packbits(np.asarray(bits, dtype=np.uint8), axis=-1, bitorder="little")


def _unpack_bits_le(b: np.ndarray, count: int) -> np.ndarray:
    return np.unpackbits(np.asarray(b, dtype=np.uint8), axis=-1, count=count,
                         bitorder="little")


def _half_bytes(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float16)
    return h.view(np.uint8).reshape(h.shape + (2,))


def write_slots_fast(k_pool: np.ndarray, v_pool: np.ndarray, slot_mapping, enc_k: dict,
                     enc_v: dict) -> None:
    """Same effect as ``write_slots`` (slots must be distinct)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    if slots.size == 0:
        return
    kc = enc_k["codes"][keep]                  # [T, H, 128]
    ks = enc_k["signs"][keep]
    vc = enc_v["codes"][keep]
    blk, off = slots // BLOCK, slots % BLOCK
    T, H = kc.shape[:2]
    ar16 = np.arange(16)[None, :]
    ar2 = np.arange(2)[None, :]
    bcol = blk[:, None]
    ar4 = np.arange(4)[None, :]
    for h in range(H):
        # fields f = 0..2 (code bit-planes) and 3 (signs), 16 bytes per token,
        # 4 bytes per coordinate chunk g at 16 (16 g + t) + 4 f
        fields = [_pack_bits_le((kc[:, h, :] >> p) & 1) for p in range(3)] + [_pack_bits_le(ks[:, h, :])]
        for f, fb in enumerate(fields):                                   # fb: [T, 16]
            for g in range(4):
                k_pool[bcol, h, (16 * (16 * g + off) + 4 * f)[:, None] + ar4] = fb[:, 4 * g: 4 * g + 4]
        k_pool[bcol, h, (1024 + 2 * off)[:, None] + ar2] = _half_bytes(enc_k["norm_f16"][keep][:, h])
        k_pool[bcol, h, (1056 + 2 * off)[:, None] + ar2] = _half_bytes(enc_k["gamma_f16"][keep][:, h])
        v_pool[bcol, h, (768 + 2 * off)[:, None] + ar2] = _half_bytes(enc_v["norm_f16"][keep][:, h])
        # V planes are coordinate-major: a 16-bit word per coordinate, a bit per token.
        words = v_pool[:, h, :768].copy().view(np.uint16).reshape(-1, 3, HEAD_DIM)
        mask = (np.uint16(1) << off.astype(np.uint16)).astype(np.uint16)   # [T]
        for p in range(3):
            bitv = ((vc[:, h, :] >> p) & 1).astype(np.uint16)            # [T, 128]
            np.bitwise_and.at(words, (blk, p), (~mask)[:, None] & np.uint16(0xFFFF))
            np.bitwise_or.at(words, (blk, p), bitv * mask[:, None])
        v_pool[:, h, :768] = words.reshape(-1, 3 * HEAD_DIM).view(np.uint8)


def read_k_tokens_fast(k_pool: np.ndarray, block_row, length: int, head: int):
    """Same result as ``read_k_tokens``."""
    nb = (length + BLOCK - 1) // BLOCK
    pages = k_pool[np.asarray(block_row[:nb], dtype=np.int64), head]    # [nb, 1088]
    codes = np.zeros((nb, BLOCK, HEAD_DIM), dtype=np.uint8)
    # [nb, chunk g, token t, field f, 4 bytes] -> per field [nb, t, 16 bytes in chunk order]
    rec = pages[:, :1024].reshape(nb, 4, BLOCK, 4, 4)
    def field(f):
        return np.ascontiguousarray(np.transpose(rec[:, :, :, f, :], (0, 2, 1, 3))).reshape(nb, BLOCK, 16)
    for p in range(3):
        codes |= (_unpack_bits_le(field(p), HEAD_DIM) << p).astype(np.uint8)
    signs = _unpack_bits_le(field(3), QJL_DIM)
    n16 = pages[:, 1024:1056].copy().view(np.float16).reshape(nb, BLOCK)
    g16 = pages[:, 1056:1088].copy().view(np.float16).reshape(nb, BLOCK)
    return (codes.reshape(-1, HEAD_DIM)[:length], signs.reshape(-1, QJL_DIM)[:length],
            n16.reshape(-1)[:length], g16.reshape(-1)[:length])


def read_v_tokens_fast(v_pool: np.ndarray, block_row, length: int, head: int):
    """Same result as ``read_v_tokens``."""
    nb = (length + BLOCK - 1) // BLOCK
    pages = v_pool[np.asarray(block_row[:nb], dtype=np.int64), head]    # [nb, 800]
    codes = np.zeros((nb, BLOCK, HEAD_DIM), dtype=np.uint8)
    for p in range(3):
        raw = pages[:, 256 * p: 256 * p + 256].reshape(nb, HEAD_DIM, 2)  # [nb, dim, 2 bytes]
        bits = _unpack_bits_le(raw, BLOCK)                               # [nb, dim, token]
        codes |= (np.transpose(bits, (0, 2, 1)) << p).astype(np.uint8)
    n16 = pages[:, 768:800].copy().view(np.float16).reshape(nb, BLOCK)
    return codes.reshape(-1, HEAD_DIM)[:length], n16.reshape(-1)[:length]
