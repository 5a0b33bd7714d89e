// Fused TurboQuant encoder for gfx950.
//
// A persistent grid of 4-wave workgroups walks tiles of 16 consecutive tokens
// of one KV head; each tile encodes the 16 keys and the 16 values (SwiftLM
// README, "TurboQuantization: KV Cache Compression", K-cache steps 1-5 and the
// V-cache paragraph).
//
// Vector pass.  Wave w takes tokens 4w..4w+3; in a wave, the 16 lanes of row r
// hold token 4w+r and lane i of the row holds the 8 consecutive coordinates
// 8i..8i+7, so every input vector arrives with one 16-byte load per lane
// (narrow per-lane loads cap HBM throughput well below its peak).
//   - norm: 8 squares per lane, then a sum over the row (DPP exchanges);
//   - Walsh-Hadamard rotation: coordinate bits 0-2 are in-lane butterflies,
//     bits 3-6 pair lanes i and i^1, ^2, ^4, ^8 of the same row (DPP);
//   - codes: seven fp32 compares per coordinate ("t_j < y"), turned into the
//     three bits of the level rank; a lane's 8 coordinates give one byte of
//     each bit-plane record -- for keys exactly byte i of the token's record;
//   - keys only: residual e = y - c[idx] (rotated domain), its length, and
//     e * 2^8 (exact scaling) staged in LDS as a half "hi" part plus a half
//     "lo" remainder.
// Value planes are coordinate-major (one 16-bit word per coordinate, a bit per
// token): the per-token bytes are staged, then 8x8 bit-matrix transposes turn
// 16 tokens x 8 coordinates into 8 coordinate words.
// QJL projection (matrix cores).  z = S r with r = H^T e is z = (S H) e.  Each
// wave owns 32 of the 128 projection rows and keeps its rows of S H (hi and lo
// halves, 64 registers) for the whole run; three f16 MFMA passes
// (hi.hi + hi.lo + lo.hi) carry ~22 significant bits, so a sign differs from
// exact arithmetic only within ~1e-6 of zero.  A ballot of "z >= 0" gives
// 16-bit pieces of four tokens' sign records at once.
// Output.  A tile that fills one page in order is written as 68 + 50
// coalesced 16-byte stores from the LDS page images; otherwise records go out
// token by token and value bits are merged into their pages with 32-bit
// atomic and/or.  Barriers order LDS only, so stores stay in flight, and the
// next tile's inputs are loaded while the current one is processed.

#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kEncTokens = 16;
constexpr int kEStride = 136;  // halves per staged residual row (128 + pad: spreads LDS banks)
constexpr float kResidualScale = 256.0f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Level index of y: the number of thresholds strictly below it (a value on
// a threshold goes to the lower cell), compared in fp32.  Each compare is
// folded into the count at once, so no lane mask stays live.
__device__ __forceinline__ int level_index(float y, const Codebook &cb) {
  int idx = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) idx += (cb.t[j] < y) ? 1 : 0;
  return idx;
}

// 8 coordinates of one vector as raw bytes: one 16-byte load (bf16, f16) or
// two (fp32).
struct Raw8 {
  uint4 a, b;
};

__device__ __forceinline__ Raw8 load_raw8(const void *base, int dtype, int64_t elem) {
  Raw8 r;
  if (dtype == TQ_F32) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + elem);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
    r.b = make_uint4(0u, 0u, 0u, 0u);
  }
  return r;
}

__device__ __forceinline__ void unpack8(const Raw8 &r, int dtype, float (&x)[8]) {
  if (dtype == TQ_F32) {
    x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y);
    x[2] = __uint_as_float(r.a.z); x[3] = __uint_as_float(r.a.w);
    x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y);
    x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
  } else {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (dtype == TQ_BF16) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      } else {
        x[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xFFFFu));
        x[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
      }
    }
  }
}

// Sum over the 16 lanes of a row, in every lane of the row.
__device__ __forceinline__ float row_sum(float v) {
  v += xchg1(v);
  v += xchg2(v);
  v += xchg4(v);
  v += xchg8(v);
  return v;
}

// Unnormalised Walsh-Hadamard transform of a 128-vector spread over one row:
// lane i holds coordinates 8i..8i+7.  Bits 0-2 of the coordinate are in-lane,
// bits 3-6 are lane bits 0-3 (butterfly partner = lane ^ s, kept in the row).
__device__ __forceinline__ void row_fwht(float (&x)[8], int lane) {
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & s) continue;
      const float a = x[j], b = x[j + s];
      x[j] = a + b;
      x[j + s] = a - b;
    }
  }
#pragma unroll
  for (int s = 1; s <= 8; s <<= 1) {
    const float sg = (lane & s) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fmaf(sg, x[j], xchg(x[j], s, lane));
  }
}

// 8x8 bit-matrix transpose of a 64-bit word: bit c of byte r moves to bit r
// of byte c (three shift-and-mask exchange steps).
__device__ __forceinline__ uint64_t transpose8x8(uint64_t x) {
  uint64_t t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
  x = x ^ t ^ (t << 7);
  t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
  x = x ^ t ^ (t << 14);
  t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
  x = x ^ t ^ (t << 28);
  return x;
}

__device__ __forceinline__ half8 load_half8(const uint16_t *p) {
  return *reinterpret_cast<const half8 *>(p);
}

__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a, int64_t num_tiles) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane >> 4, oct = lane & 15;   // token 4*wave+row, coordinates 8*oct..+7
  const int H = a.num_kv_heads;
  const int tok = 4 * wave + row;

  __shared__ __align__(16) _Float16 ehi[kEncTokens][kEStride];
  __shared__ __align__(16) _Float16 elo[kEncTokens][kEStride];
  __shared__ __align__(16) uint8_t kst[kKPage];               // K page image, by tile position
  __shared__ __align__(16) uint8_t vst[3][16][kEncTokens];    // V plane bytes [plane][octet][token]
  __shared__ __align__(16) uint16_t vwords[3][kHeadDim];      // V words, bit t = tile token t
  __shared__ __align__(16) uint16_t vnorm[kEncTokens];
  __shared__ int blk[kEncTokens], off[kEncTokens], valid[kEncTokens], leader[kEncTokens];
  __shared__ int full_page;
  __shared__ float lut[8];

  if (tid < 8) {
    float cv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cv[j] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.c[j])));
    float c = cv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) c = (tid == j) ? cv[j] : c;
    lut[tid] = c;
  }

  // This wave's projection rows: 16 * (2 * wave + nt) + (lane % 16), columns
  // 32 * kk + 8 * (lane / 16) + 0..7 -- the B operand layout of the f16 MFMA.
  half8 bhi[2][4], blo[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int prow = 16 * (2 * wave + nt) + (lane & 15);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int col = 32 * kk + 8 * (lane >> 4);
      bhi[nt][kk] = load_half8(a.SHhi + prow * kHeadDim + col);
      blo[nt][kk] = load_half8(a.SHlo + prow * kHeadDim + col);
    }
  }

  // Software pipeline: slot and raw inputs of this lane's token for the next
  // tile are loaded while the current tile is processed.
  auto load_tile = [&](int64_t tl, int64_t &slot, Raw8 &rk, Raw8 &rv) {
    const int hh = (int)(tl % H);
    const int64_t tb = (tl / H) * kEncTokens;
    slot = -1;
    if (tid < kEncTokens && tb + tid < a.num_tokens) slot = a.slots[tb + tid];
    const int64_t t = tb + tok;
    rk.a = rk.b = rv.a = rv.b = make_uint4(0u, 0u, 0u, 0u);
    if (t < a.num_tokens) {
      const int64_t e = t * a.tok_stride + (int64_t)hh * a.head_stride + 8 * oct;
      rk = load_raw8(a.k, a.dtype, e);
      rv = load_raw8(a.v, a.dtype, e);
    }
  };
  int64_t slot_cur = -1;
  Raw8 rk_cur, rv_cur;
  rk_cur.a = rk_cur.b = rv_cur.a = rv_cur.b = make_uint4(0u, 0u, 0u, 0u);
  if ((int64_t)blockIdx.x < num_tiles) load_tile(blockIdx.x, slot_cur, rk_cur, rv_cur);

  for (int64_t tile = blockIdx.x; tile < num_tiles; tile += gridDim.x) {
    const int h = (int)(tile % H);
    const int64_t t0 = (tile / H) * kEncTokens;

    if (tid < kEncTokens) {
      valid[tid] = slot_cur >= 0;
      blk[tid] = slot_cur >= 0 ? (int)(slot_cur / kBlock) : -1;
      off[tid] = slot_cur >= 0 ? (int)(slot_cur % kBlock) : 0;
    }
    lds_barrier();
    if (tid < kEncTokens) {
      int lead = valid[tid];
      for (int u = 0; u < tid; ++u)
        if (valid[u] && blk[u] == blk[tid]) lead = 0;
      leader[tid] = lead;
    }
    if (tid == 32) {
      int full = 1;
      for (int u = 0; u < kEncTokens; ++u)
        full &= valid[u] && blk[u] == blk[0] && off[u] == u;
      full_page = full;
    }
    int64_t slot_next = -1;
    Raw8 rk_next, rv_next;
    rk_next.a = rk_next.b = rv_next.a = rv_next.b = make_uint4(0u, 0u, 0u, 0u);
    const int64_t next = tile + gridDim.x;
    if (next < num_tiles) load_tile(next, slot_next, rk_next, rv_next);

    // ---- vector pass: keys and values of token `tok`, 8 coordinates a lane ---
    {
      float xk[8], xv[8];
      unpack8(rk_cur, a.dtype, xk);
      unpack8(rv_cur, a.dtype, xv);
      float qk = 0.0f, qv = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qk = fmaf(xk[j], xk[j], qk);
        qv = fmaf(xv[j], xv[j], qv);
      }
      const float nk = sqrtf(row_sum(qk)), nv = sqrtf(row_sum(qv));
      row_fwht(xk, lane);
      row_fwht(xv, lane);
      const float sk = nk > 0.0f ? kInvSqrt128 / nk : 0.0f;
      const float sv = nv > 0.0f ? kInvSqrt128 / nv : 0.0f;

      int kb[3] = {0, 0, 0}, vb[3] = {0, 0, 0};
      float e[8];
      float ge = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float yk = xk[j] * sk, yv = xv[j] * sv;
        const int bk = level_index(yk, a.cb), bv = level_index(yv, a.cb);
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          kb[p] |= ((bk >> p) & 1) << j;
          vb[p] |= ((bv >> p) & 1) << j;
        }
        e[j] = yk - lut[bk];
        ge = fmaf(e[j], e[j], ge);
      }
      const float gam = sqrtf(row_sum(ge));
      if (valid[tok]) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          kst[kKPlane * p + 16 * tok + oct] = (uint8_t)kb[p];
          vst[p][oct][tok] = (uint8_t)vb[p];
        }
        half8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float s = e[j] * kResidualScale;
          hi[j] = (_Float16)s;
          lo[j] = (_Float16)(s - (float)hi[j]);
        }
        *reinterpret_cast<half8 *>(&ehi[tok][8 * oct]) = hi;
        *reinterpret_cast<half8 *>(&elo[tok][8 * oct]) = lo;
        if (oct == 0) {
          *reinterpret_cast<_Float16 *>(kst + kKNorm + 2 * tok) = to_half_sat(nk);
          *reinterpret_cast<_Float16 *>(kst + kKGamma + 2 * tok) = to_half_sat(gam);
          vnorm[tok] = __builtin_bit_cast(uint16_t, to_half_sat(nv));
          if (a.norms_out) {
            float *no = a.norms_out + ((t0 + tok) * H + h) * 3;
            no[0] = nk;
            no[1] = gam;
            no[2] = nv;
          }
        }
      } else {
#pragma unroll
        for (int p = 0; p < 3; ++p) vst[p][oct][tok] = 0;
      }
    }
    lds_barrier();

    // ---- value words: 16 tokens x 8 coordinates -> 8 coordinate words -------
    if (tid < 48) {
      const int p = tid >> 4, c8 = tid & 15;
      const uint64_t lo = transpose8x8(*reinterpret_cast<const uint64_t *>(&vst[p][c8][0]));
      const uint64_t hi = transpose8x8(*reinterpret_cast<const uint64_t *>(&vst[p][c8][8]));
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = (uint32_t)((lo >> (16 * q)) & 0xFFu) | ((uint32_t)((hi >> (16 * q)) & 0xFFu) << 8);
        const uint32_t w1 = (uint32_t)((lo >> (16 * q + 8)) & 0xFFu) | ((uint32_t)((hi >> (16 * q + 8)) & 0xFFu) << 8);
        w[q] = w0 | (w1 << 16);
      }
      *reinterpret_cast<uint4 *>(&vwords[p][8 * c8]) = make_uint4(w[0], w[1], w[2], w[3]);
    }

    // ---- QJL projection on the matrix cores --------------------------------
    {
      const int arow = lane & 15, acol = 8 * (lane >> 4);
      float4v acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8 ah = *reinterpret_cast<const half8 *>(&ehi[arow][32 * kk + acol]);
        const half8 al = *reinterpret_cast<const half8 *>(&elo[arow][32 * kk + acol]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bhi[nt][kk], acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, blo[nt][kk], acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bhi[nt][kk], acc[nt], 0, 0, 0);
        }
      }
      // acc[nt][i] at lane l is z for token 4*(l/16)+i, row 16*(2*wave+nt) + l%16
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t bits = __ballot(acc[nt][i] >= 0.0f);
          if (lane < 4)
            *reinterpret_cast<uint16_t *>(kst + kKSigns + 16 * (4 * lane + i) + 2 * (2 * wave + nt)) =
                (uint16_t)(bits >> (16 * lane));
        }
      }
    }
    lds_barrier();

    // ---- write the tile out ------------------------------------------------
    if (full_page) {
      // one page each: K as 68 and V as 50 coalesced 16-byte stores
      uint8_t *kp = a.k_cache + ((int64_t)blk[0] * H + h) * kKPage;
      uint8_t *vp = a.v_cache + ((int64_t)blk[0] * H + h) * kVPage;
      if (tid < kKPage / 16) {
        *reinterpret_cast<uint4 *>(kp + 16 * tid) = *reinterpret_cast<const uint4 *>(kst + 16 * tid);
      } else if (tid < kKPage / 16 + 48) {
        const int q = tid - kKPage / 16;
        *reinterpret_cast<uint4 *>(vp + 16 * q) =
            *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(vwords) + 16 * q);
      } else if (tid < kKPage / 16 + 50) {
        const int q = tid - kKPage / 16 - 48;
        *reinterpret_cast<uint4 *>(vp + kVNorm + 16 * q) =
            *reinterpret_cast<const uint4 *>(&vnorm[8 * q]);
      }
    } else {
      // token by token: K records (3 planes + signs as 16-byte pieces, two
      // halves), the V norm, and V bits merged into their pages atomically
      if (tid < 4 * kEncTokens) {
        const int n = tid >> 2, piece = tid & 3;
        if (valid[n]) {
          uint8_t *kp = a.k_cache + ((int64_t)blk[n] * H + h) * kKPage;
          const int src = piece < 3 ? kKPlane * piece + 16 * n : kKSigns + 16 * n;
          const int dst = piece < 3 ? kKPlane * piece + 16 * off[n] : kKSigns + 16 * off[n];
          *reinterpret_cast<uint4 *>(kp + dst) = *reinterpret_cast<const uint4 *>(kst + src);
        }
      } else if (tid < 5 * kEncTokens) {
        const int n = tid - 4 * kEncTokens;
        if (valid[n]) {
          uint8_t *kp = a.k_cache + ((int64_t)blk[n] * H + h) * kKPage;
          uint8_t *vp = a.v_cache + ((int64_t)blk[n] * H + h) * kVPage;
          *reinterpret_cast<uint16_t *>(kp + kKNorm + 2 * off[n]) =
              *reinterpret_cast<const uint16_t *>(kst + kKNorm + 2 * n);
          *reinterpret_cast<uint16_t *>(kp + kKGamma + 2 * off[n]) =
              *reinterpret_cast<const uint16_t *>(kst + kKGamma + 2 * n);
          *reinterpret_cast<uint16_t *>(vp + kVNorm + 2 * off[n]) = vnorm[n];
        }
      }
      for (int w = tid; w < 3 * kHeadDim; w += 256) {
        const int p = w / kHeadDim, i = w % kHeadDim;
        const uint32_t word = vwords[p][i];
        for (int j = 0; j < kEncTokens; ++j) {
          if (!leader[j]) continue;
          uint32_t mask = 0, bits = 0;
          for (int u = j; u < kEncTokens; ++u) {
            if (valid[u] && blk[u] == blk[j]) {
              mask |= 1u << off[u];
              bits |= ((word >> u) & 1u) << off[u];
            }
          }
          uint8_t *vp = a.v_cache + ((int64_t)blk[j] * H + h) * kVPage;
          const uintptr_t addr = reinterpret_cast<uintptr_t>(vp + kKPlane * p + 2 * i);
          uint32_t *w32 = reinterpret_cast<uint32_t *>(addr & ~uintptr_t(3));
          const int sh = (addr & 2) ? 16 : 0;
          const uint32_t set = bits << sh, clr = (mask & ~bits) << sh;
          if (clr) atomicAnd(w32, ~clr);
          if (set) atomicOr(w32, set);
        }
      }
    }
    lds_barrier();  // LDS tile state is rewritten by the next iteration
    slot_cur = slot_next;
    rk_cur = rk_next;
    rv_cur = rv_next;
  }
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream) {
  const int64_t groups = (a.num_tokens + kEncTokens - 1) / kEncTokens;
  const int64_t tiles = groups * a.num_kv_heads;
  const int64_t grid = tiles < 1024 ? tiles : 1024;  // persistent: ~4 workgroups per CU
  hipLaunchKernelGGL(encode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a, tiles);
  return hipGetLastError();
}

}  // namespace tq
