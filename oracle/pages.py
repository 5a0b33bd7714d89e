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

For b-bit codes (b = 2, 3, 4; the pages' method uses b = 3), with
RB = 4 (b + 1) bytes per record:
K page (256 (b + 1) + 64 B; 1088 for b = 3):
  [0, 64 RB)    : 64 records of RB bytes, chunk-major: the record of
      coordinate chunk g = 0..3 (coordinates 32g .. 32g + 31) and token t is
      at RB (16 g + t); its little-endian 32-bit words are field
      f = 0 .. b-1 (code bit-plane f: bit i % 32 of the word holds bit f of
      code_i for coordinate i = 32 g + i % 32) and f = b (QJL signs: bit
      i % 32 holds the sign bit of projection row i = 32 g + i % 32; 1 means
      z_i >= 0).  So bit f of code_i / the sign of row i sits at byte
      RB (16 (i // 32) + t) + 4 f + (i % 32) // 8, bit i % 8.
  [64 RB, 64 RB + 32)      : half n_t at 64 RB + 2t.
  [64 RB + 32, 64 RB + 64) : half gamma_t at 64 RB + 32 + 2t.
V page (256 b + 32 B; 800 for b = 3):
  [256p, 256p + 256), p = 0 .. b-1 : code bit-plane p, coordinate-major:
      coordinate i owns the 16-bit word at 256p + 2i; its bit t holds bit p
      of token t's code for coordinate i.
  [256 b, 256 b + 32) : half n_t at 256 b + 2t.
The functions below take the bit width from the page (or pool) size.
Bits per coordinate: 1088*8/(16*128) = 4.25 and 800*8/(16*128) = 3.125.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16
HEAD_DIM = 128
QJL_DIM = 128


def k_record_bytes(bits: int) -> int:
    return 4 * (bits + 1)


def k_page_bytes(bits: int) -> int:
    return 64 * k_record_bytes(bits) + 2 * BLOCK + 2 * BLOCK


def v_page_bytes(bits: int) -> int:
    return 256 * bits + 2 * BLOCK


def k_norm_offset(bits: int) -> int:
    return 64 * k_record_bytes(bits)


def v_norm_offset(bits: int) -> int:
    return 256 * bits


def k_page_bits(nbytes: int) -> int:
    """Bit width of a K page of ``nbytes`` bytes."""
    b = (nbytes - 4 * BLOCK) // 256 - 1
    assert k_page_bytes(b) == nbytes, nbytes
    return b


def v_page_bits(nbytes: int) -> int:
    b = (nbytes - 2 * BLOCK) // 256
    assert v_page_bytes(b) == nbytes, nbytes
    return b


K_PAGE_BYTES = k_page_bytes(3)
V_PAGE_BYTES = v_page_bytes(3)


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


def k_bit_byte(t: int, i: int, field: int, bits: int = 3) -> int:
    """Byte of the K page holding field ``field`` (0 .. bits-1: code
    bit-plane, bits: QJL sign) of coordinate / row ``i`` of token ``t``; the
    bit is i % 8."""
    return k_record_bytes(bits) * (16 * (i // 32) + t) + 4 * field + (i % 32) // 8


def set_k_slot(page: np.ndarray, t: int, codes, signs, n16, g16) -> None:
    bits = k_page_bits(page.shape[-1])
    for i in range(HEAD_DIM):
        for p in range(bits):
            _put_bit(page, k_bit_byte(t, i, p, bits), i % 8, (int(codes[i]) >> p) & 1)
    for i in range(QJL_DIM):
        _put_bit(page, k_bit_byte(t, i, bits, bits), i % 8, int(signs[i]))
    _put_half(page, k_norm_offset(bits) + 2 * t, n16)
    _put_half(page, k_norm_offset(bits) + 32 + 2 * t, g16)


def get_k_slot(page: np.ndarray, t: int):
    bits = k_page_bits(page.shape[-1])
    codes = np.zeros(HEAD_DIM, dtype=np.uint8)
    signs = np.zeros(QJL_DIM, dtype=np.uint8)
    for i in range(HEAD_DIM):
        v = 0
        for p in range(bits):
            v |= _get_bit(page, k_bit_byte(t, i, p, bits), i % 8) << p
        codes[i] = v
    for i in range(QJL_DIM):
        signs[i] = _get_bit(page, k_bit_byte(t, i, bits, bits), i % 8)
    no = k_norm_offset(bits)
    return codes, signs, _get_half(page, no + 2 * t), _get_half(page, no + 32 + 2 * t)


def set_v_slot(page: np.ndarray, t: int, codes, n16) -> None:
    bits = v_page_bits(page.shape[-1])
    for i in range(HEAD_DIM):
        for p in range(bits):
            word = 256 * p + 2 * i
            _put_bit(page, word + t // 8, t % 8, (int(codes[i]) >> p) & 1)
    _put_half(page, v_norm_offset(bits) + 2 * t, n16)


def get_v_slot(page: np.ndarray, t: int):
    bits = v_page_bits(page.shape[-1])
    codes = np.zeros(HEAD_DIM, dtype=np.uint8)
    for i in range(HEAD_DIM):
        v = 0
        for p in range(bits):
            v |= _get_bit(page, 256 * p + 2 * i + t // 8, t % 8) << p
        codes[i] = v
    return codes, _get_half(page, v_norm_offset(bits) + 2 * t)


def pack_k_page(codes, signs, n16, g16, bits: int = 3) -> np.ndarray:
    """One full K page from ``codes[16][128]``, ``signs[16][128]``, halves."""
    page = np.zeros(k_page_bytes(bits), dtype=np.uint8)
    for t in range(BLOCK):
        set_k_slot(page, t, codes[t], signs[t], n16[t], g16[t])
    return page


def unpack_k_page(page: np.ndarray):
    out = [get_k_slot(page, t) for t in range(BLOCK)]
    return (np.stack([o[0] for o in out]), np.stack([o[1] for o in out]),
            np.array([o[2] for o in out], dtype=np.float16),
            np.array([o[3] for o in out], dtype=np.float16))


def pack_v_page(codes, n16, bits: int = 3) -> np.ndarray:
    page = np.zeros(v_page_bytes(bits), dtype=np.uint8)
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
    bits = k_page_bits(k_pool.shape[-1])
    assert v_page_bits(v_pool.shape[-1]) == bits
    RB, kn, vn = k_record_bytes(bits), k_norm_offset(bits), v_norm_offset(bits)
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
    ar2 = np.arange(2)[None, :]
    bcol = blk[:, None]
    ar4 = np.arange(4)[None, :]
    for h in range(H):
        # fields f = 0 .. bits-1 (code bit-planes) and bits (signs), RB bytes
        # per token, 4 bytes per coordinate chunk g at RB (16 g + t) + 4 f
        fields = [_pack_bits_le((kc[:, h, :] >> p) & 1) for p in range(bits)] + [_pack_bits_le(ks[:, h, :])]
        for f, fb in enumerate(fields):                                   # fb: [T, 16]
            for g in range(4):
                k_pool[bcol, h, (RB * (16 * g + off) + 4 * f)[:, None] + ar4] = fb[:, 4 * g: 4 * g + 4]
        k_pool[bcol, h, (kn + 2 * off)[:, None] + ar2] = _half_bytes(enc_k["norm_f16"][keep][:, h])
        k_pool[bcol, h, (kn + 32 + 2 * off)[:, None] + ar2] = _half_bytes(enc_k["gamma_f16"][keep][:, h])
        v_pool[bcol, h, (vn + 2 * off)[:, None] + ar2] = _half_bytes(enc_v["norm_f16"][keep][:, h])
        # V planes are coordinate-major: a 16-bit word per coordinate, a bit per token.
        words = v_pool[:, h, :vn].copy().view(np.uint16).reshape(-1, bits, HEAD_DIM)
        mask = (np.uint16(1) << off.astype(np.uint16)).astype(np.uint16)   # [T]
        for p in range(bits):
            bitv = ((vc[:, h, :] >> p) & 1).astype(np.uint16)            # [T, 128]
            np.bitwise_and.at(words, (blk, p), (~mask)[:, None] & np.uint16(0xFFFF))
            np.bitwise_or.at(words, (blk, p), bitv * mask[:, None])
        v_pool[:, h, :vn] = words.reshape(-1, bits * HEAD_DIM).view(np.uint8)


def read_k_tokens_fast(k_pool: np.ndarray, block_row, length: int, head: int):
    """Same result as ``read_k_tokens``."""
    bits = k_page_bits(k_pool.shape[-1])
    RB, kn = k_record_bytes(bits), k_norm_offset(bits)
    nb = (length + BLOCK - 1) // BLOCK
    pages = k_pool[np.asarray(block_row[:nb], dtype=np.int64), head]    # [nb, page bytes]
    codes = np.zeros((nb, BLOCK, HEAD_DIM), dtype=np.uint8)
    # [nb, chunk g, token t, field f, 4 bytes] -> per field [nb, t, 16 bytes in chunk order]
    rec = pages[:, :kn].reshape(nb, 4, BLOCK, bits + 1, 4)
    def field(f):
        return np.ascontiguousarray(np.transpose(rec[:, :, :, f, :], (0, 2, 1, 3))).reshape(nb, BLOCK, 16)
    for p in range(bits):
        codes |= (_unpack_bits_le(field(p), HEAD_DIM) << p).astype(np.uint8)
    signs = _unpack_bits_le(field(bits), QJL_DIM)
    n16 = pages[:, kn:kn + 32].copy().view(np.float16).reshape(nb, BLOCK)
    g16 = pages[:, kn + 32:kn + 64].copy().view(np.float16).reshape(nb, BLOCK)
    return (codes.reshape(-1, HEAD_DIM)[:length], signs.reshape(-1, QJL_DIM)[:length],
            n16.reshape(-1)[:length], g16.reshape(-1)[:length])


def read_v_tokens_fast(v_pool: np.ndarray, block_row, length: int, head: int):
    """Same result as ``read_v_tokens``."""
    bits = v_page_bits(v_pool.shape[-1])
    vn = v_norm_offset(bits)
    nb = (length + BLOCK - 1) // BLOCK
    pages = v_pool[np.asarray(block_row[:nb], dtype=np.int64), head]    # [nb, page bytes]
    codes = np.zeros((nb, BLOCK, HEAD_DIM), dtype=np.uint8)
    for p in range(bits):
        raw = pages[:, 256 * p: 256 * p + 256].reshape(nb, HEAD_DIM, 2)  # [nb, dim, 2 bytes]
        bits_t = _unpack_bits_le(raw, BLOCK)                             # [nb, dim, token]
        codes |= (np.transpose(bits_t, (0, 2, 1)) << p).astype(np.uint8)
    n16 = pages[:, vn:vn + 32].copy().view(np.float16).reshape(nb, BLOCK)
    return codes.reshape(-1, HEAD_DIM)[:length], n16.reshape(-1)[:length]
