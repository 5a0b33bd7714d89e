// Fused TurboQuant encoder for gfx950 (SwiftLM README, "TurboQuantization: KV
// Cache Compression": K-cache steps 1-5 and the V-cache paragraph).
//
// A persistent grid of 4-wave workgroups walks rounds of four tiles; a tile
// is 16 consecutive tokens of one KV head and wave w owns tile w of a round.
//
// Rotation on the matrix cores.  The Walsh-Hadamard transform is a product
// with H_128 = H_8 (x) H_16 (Sylvester, entries +-1), exact in bf16/f16, so
// y = H x runs as 16x16x32 MFMAs on the raw inputs (fp32 inputs as three bf16
// pieces).  Every 16x32 block of H is one of four +-1 register sets (the rows
// of H_16 with the sign of an H_8 entry, which may flip between the two lane
// halves).  Keys use C = X H (rows = tokens), values C = H X^T (rows =
// coordinates), so both read the same 16-byte input loads.
//
// Codes from wave masks.  With the symmetric codebook, the level rank is
// idx = [y > 0] ? 4 + c : 3 - c, c = #{k : t_k < |y|} over the three positive
// thresholds (a tie goes to the lower cell for either sign, as #{t_j < y}).
// Comparing |y| with t_k * ||y_raw|| gives the masks A_k (thermometer code)
// and P = [y > 0]; the bit-planes are b2 = P, b1 = ~(A2 ^ P),
// b0 = ~(A1 ^ A2 ^ A3 ^ P).  A mask of a key MFMA register covers 16 coordinates
// of four tokens and of a value register 16 tokens of four coordinates: in
// both cases 16-bit pieces of the page layout, moved out with writelane.
//
// Keys: residual e = y - c[idx] (rotated domain), gamma = ||e||, and the QJL
// projection z = S r = (S H) e (r = H^T e) on the f16 MFMA with e and S H as
// hi + lo halves (three passes, ~22 bits).  Wave w computes rows
// 32w .. 32w+31 of z for all four tiles of the round from e staged in LDS;
// a mask of "z >= 0" is a 16-bit piece of four tokens' sign records.
//
// Output: a tile that fills one page in order is written with coalesced
// 16-byte stores of the LDS page images; otherwise records go out token by
// token and value bits are merged into their pages with 32-bit atomic and/or.

#include <utility>

#include "tq_common.hpp"
#include "tq_append.hpp"

namespace tq {
namespace {

constexpr int kTok = 16;          // tokens per tile
constexpr int kTiles = 4;         // tiles per round (one per wave)
constexpr int kEHalves = 136;     // halves per staged residual row (128 + pad: spreads LDS banks)
constexpr float kResScale = 256.0f;
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maximum

typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int parity(uint32_t x) { return __builtin_popcount(x) & 1; }

// The four +-1 operand sets (8 values of 16 bits a lane).  Lane l holds
// H_16[8*((l/16)&1) + j][l%16] for j = 0..7, as +-one.  Set 0: as is; 1: negated;
// 2: negated in lanes 32..63; 3: negated in lanes 0..31.
struct HSets {
  v8s s[4];
};

__device__ __forceinline__ HSets make_hsets(int lane, uint16_t one) {
  HSets h;
  const int l16 = lane & 15, half = (lane >> 4) & 1, upper = lane >= 32;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t b = parity((uint32_t)((8 * half + j) & l16)) ? (uint16_t)(one | 0x8000u) : one;
    h.s[0][j] = (short)b;
    h.s[1][j] = (short)(b ^ 0x8000u);
    h.s[2][j] = (short)(upper ? (b ^ 0x8000u) : b);
    h.s[3][j] = (short)(upper ? b : (b ^ 0x8000u));
  }
  return h;
}

// Operand for K step k (input coordinates 32k..32k+31) and output block n
// (coordinates 16n..16n+15): H[32k + 8(l/16) + j][16n + l%16] =
// H_8[2k + (l >= 32)][n] * H_16[...] -- the lane-half sign is a compile-time
// function of (k, n).
__device__ __forceinline__ const v8s &hop(const HSets &h, int k, int n) {
  const int s0 = parity((uint32_t)((2 * k) & n)), s1 = parity((uint32_t)((2 * k + 1) & n));
  if (s0 == s1) return s0 ? h.s[1] : h.s[0];
  return s0 ? h.s[3] : h.s[2];
}

template <bool F16>
__device__ __forceinline__ v4f mfma16(const v8s &a, const v8s &b, const v4f &c) {
  if (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) uint32_t gword;

// Raw inputs of one lane: token l%16, coordinates 32k + 8(l/16) .. +7 for
// k = 0..3, as loaded (16 bytes per k for 16-bit inputs, 32 for fp32).
template <int PC>
struct In {
  u32x4 w[4][PC == 3 ? 2 : 1];
};

// bf16 pieces hi + mid + lo of a float (exact for normal values).
struct Split3 {
  short h, m, l;
};
__device__ __forceinline__ Split3 split3(float v) {
  const __bf16 bh = (__bf16)v;
  const float r1 = v - (float)bh;
  const __bf16 bm = (__bf16)r1;
  const float r2 = r1 - (float)bm;
  const __bf16 bl = (__bf16)r2;
  return {__builtin_bit_cast(short, bh), __builtin_bit_cast(short, bm), __builtin_bit_cast(short, bl)};
}

template <int PC>
__device__ __forceinline__ void load_in(In<PC> &r, const void *base, int64_t elem0) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (PC == 1) {
      r.w[k][0] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + elem0 + 32 * k);
    } else {
      const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + elem0 + 32 * k);
      r.w[k][0] = p[0];
      r.w[k][1] = p[1];
    }
  }
}

// Matrix operands of the raw inputs: 16-bit values as they are, fp32 as
// three bf16 pieces.  Converted where they are used, so that the loads of a
// prefetched round are not waited for when they are issued.
template <int PC>
__device__ __forceinline__ void pieces(const In<PC> &r, v8s (&x)[4][PC]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (PC == 1) {
      x[k][0] = __builtin_bit_cast(v8s, r.w[k][0]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const Split3 sp = split3(__uint_as_float(r.w[k][j >> 2][j & 3]));
        x[k][0][j] = sp.h;
        x[k][1][j] = sp.m;
        x[k][2][j] = sp.l;
      }
    }
  }
}

// Per round LDS state (pages of BITS-bit codes).
template <int BITS>
struct RoundLds {
  uint8_t kimg[kTiles][k_page_bytes(BITS)];     // K page images
  uint8_t vimg[kTiles][v_page_bytes(BITS)];     // V page images
  _Float16 ehi[kTiles][kTok][kEHalves];         // residual * 256 (hi), slot order
  _Float16 elo[kTiles][kTok][kEHalves];         // remainder (lo)
  int blk[kTiles][kTok], off[kTiles][kTok], valid[kTiles][kTok];
  float nout[kTiles][kTok][3];                  // n_K, gamma, n_V in fp32 (optional output)
  int full[kTiles];
  int active[kTiles];
};

// v_writelane_b32 through the LLVM intrinsic (HIP exposes no builtin for it):
// the compiler then sees the scalar read and inserts the wait states a
// preceding compare that wrote the mask requires, which it cannot do for
// hand-written assembly.
extern "C" __device__ int tq_llvm_writelane(int val, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Lane LANE of v takes the uniform value s.
template <int LANE>
__device__ __forceinline__ void writelane(uint32_t &v, uint32_t s) {
  v = (uint32_t)tq_llvm_writelane((int)s, LANE, (int)v);
}
// Moves a 64-bit wave mask into lanes 2Q (bits 0-31) and 2Q+1 (bits 32-63) of v.
template <int Q>
__device__ __forceinline__ void put_mask(uint32_t &v, uint64_t m) {
  writelane<2 * Q>(v, (uint32_t)m);
  writelane<2 * Q + 1>(v, (uint32_t)(m >> 32));
}

// The unrolled steps below are template functions of their step number with
// scalar arguments by value (not closures): a closure holding references to
// the levels turns a select between levels into an indexed load and keeps
// everything it captures in scratch memory.

// Value masks of register (m, i) = 4m + i of C = H X^T: lanes of coordinate
// 16m + 4(l/16) + i, token l%16.
template <int Q>
__device__ __forceinline__ void value_step(const v4f (&vy)[8], float T0, float T1, float T2, uint32_t (&vb)[3]) {
  constexpr int m = Q >> 2, i = Q & 3;
  const float y = vy[m][i];
  const uint64_t A1 = __ballot(fabsf(y) > T0), A2 = __ballot(fabsf(y) > T1);
  const uint64_t A3 = __ballot(fabsf(y) > T2), P = __ballot(y > 0.0f);
  put_mask<Q>(vb[0], ~(A1 ^ A2 ^ A3 ^ P));
  put_mask<Q>(vb[1], ~(A2 ^ P));
  put_mask<Q>(vb[2], P);
}
template <int... Q>
__device__ __forceinline__ void value_steps(std::integer_sequence<int, Q...>, const v4f (&vy)[8], float T0, float T1,
                                            float T2, uint32_t (&vb)[3]) {
  (value_step<Q>(vy, T0, T1, T2, vb), ...);
}

// Key masks and residual of register (n, i) = 4n + i of C = X H: lanes of
// token 4(l/16) + i, coordinate 16n + l%16.  e * 256 = y * 256 / |y_raw| -
// sign * 256 * level, with thresholds T = t_k |y_raw| of the lane's token.
template <int Q>
__device__ __forceinline__ void key_step(const v4f (&ky)[8], const float (&T)[4][3], const float (&r256)[4], float c0,
                                         float c1, float c2, float c3, uint32_t (&kb)[3], float (&es)[8][4],
                                         float (&g2)[4]) {
  constexpr int n = Q >> 2, i = Q & 3;
  const float y = ky[n][i], ay = fabsf(y);
  const bool a1 = ay > T[i][0], a2 = ay > T[i][1], a3 = ay > T[i][2], pp = y > 0.0f;
  const uint64_t A1 = __ballot(a1), A2 = __ballot(a2), A3 = __ballot(a3), P = __ballot(pp);
  put_mask<Q>(kb[0], ~(A1 ^ A2 ^ A3 ^ P));
  put_mask<Q>(kb[1], ~(A2 ^ P));
  put_mask<Q>(kb[2], P);
  float lv = a1 ? c1 : c0;
  lv = a2 ? c2 : lv;
  lv = a3 ? c3 : lv;
  const float e = fmaf(y, r256[i], pp ? -lv : lv);
  es[n][i] = e;
  g2[i] = fmaf(e, e, g2[i]);
}
template <int... Q>
__device__ __forceinline__ void key_steps(std::integer_sequence<int, Q...>, const v4f (&ky)[8], const float (&T)[4][3],
                                          const float (&r256)[4], float c0, float c1, float c2, float c3,
                                          uint32_t (&kb)[3], float (&es)[8][4], float (&g2)[4]) {
  (key_step<Q>(ky, T, r256, c0, c1, c2, c3, kb, es, g2), ...);
}

// Other code widths (2 and 4 bits) take the same steps with NT = 2^(B-1) - 1
// positive thresholds: c = #{k : t_k < |y|} in thermometer masks A_1..A_NT,
// and bit p of c is the xor of the A_j with 2^p | j (floor(c / 2^p) counts
// them), so plane p < B - 1 of the rank is ~(P ^ that xor) and plane B - 1 is P.
template <int B>
__device__ __forceinline__ void code_masks(const uint64_t (&A)[(1 << (B - 1)) - 1], uint64_t P, uint64_t (&pl)[B]) {
  constexpr int NT = (1 << (B - 1)) - 1;
#pragma unroll
  for (int p = 0; p < B - 1; ++p) {
    uint64_t x = P;
#pragma unroll
    for (int j = 1; j <= NT; ++j)
      if (j % (1 << p) == 0) x ^= A[j - 1];
    pl[p] = ~x;
  }
  pl[B - 1] = P;
}
template <int B, int Q>
__device__ __forceinline__ void value_step_b(const v4f (&vy)[8], const float (&T)[(1 << (B - 1)) - 1],
                                             uint32_t (&vb)[B]) {
  constexpr int m = Q >> 2, i = Q & 3, NT = (1 << (B - 1)) - 1;
  const float y = vy[m][i], ay = fabsf(y);
  uint64_t A[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) A[k] = __ballot(ay > T[k]);
  uint64_t pl[B];
  code_masks<B>(A, __ballot(y > 0.0f), pl);
#pragma unroll
  for (int p = 0; p < B; ++p) put_mask<Q>(vb[p], pl[p]);
}
template <int B, int... Q>
__device__ __forceinline__ void value_steps_b(std::integer_sequence<int, Q...>, const v4f (&vy)[8],
                                              const float (&T)[(1 << (B - 1)) - 1], uint32_t (&vb)[B]) {
  (value_step_b<B, Q>(vy, T, vb), ...);
}
template <int B, int Q>
__device__ __forceinline__ void key_step_b(const v4f (&ky)[8], const float (&T)[4][(1 << (B - 1)) - 1],
                                           const float (&r256)[4], const float (&cp)[1 << (B - 1)], uint32_t (&kb)[B],
                                           float (&es)[8][4], float (&g2)[4]) {
  constexpr int n = Q >> 2, i = Q & 3, NT = (1 << (B - 1)) - 1;
  const float y = ky[n][i], ay = fabsf(y);
  const bool pp = y > 0.0f;
  uint64_t A[NT];
  float lv = cp[0];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const bool ak = ay > T[i][k];
    A[k] = __ballot(ak);
    lv = ak ? cp[k + 1] : lv;
  }
  uint64_t pl[B];
  code_masks<B>(A, __ballot(pp), pl);
#pragma unroll
  for (int p = 0; p < B; ++p) put_mask<Q>(kb[p], pl[p]);
  const float e = fmaf(y, r256[i], pp ? -lv : lv);
  es[n][i] = e;
  g2[i] = fmaf(e, e, g2[i]);
}
template <int B, int... Q>
__device__ __forceinline__ void key_steps_b(std::integer_sequence<int, Q...>, const v4f (&ky)[8],
                                            const float (&T)[4][(1 << (B - 1)) - 1], const float (&r256)[4],
                                            const float (&cp)[1 << (B - 1)], uint32_t (&kb)[B], float (&es)[8][4],
                                            float (&g2)[4]) {
  (key_step_b<B, Q>(ky, T, r256, cp, kb, es, g2), ...);
}

// Sign masks of register (u, i) = 4u + i of the projection of tile TL: lanes
// of token 4(l/16) + i, row 16(2w + u) + l%16.
template <int TL, int... Q>
__device__ __forceinline__ void sign_masks(std::integer_sequence<int, Q...>, const v4f (&z)[2], uint32_t &sbits) {
  (put_mask<8 * TL + Q>(sbits, __ballot(z[Q >> 2][Q & 3] >= 0.0f)), ...);
}

// Rows 32w .. 32w+31 of z = (S H) e for tile TL of the round: three f16
// passes (e_hi S_hi + e_hi S_lo + e_lo S_hi) per K step, then its sign masks.
template <int TL, int BITS>
__device__ __forceinline__ void qjl_tile(const RoundLds<BITS> &L, int l16, int lg, const v8s (&shi)[2][4],
                                         const v8s (&slo)[2][4], uint32_t &sbits) {
  v4f z[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const v8h ah = *reinterpret_cast<const v8h *>(&L.ehi[TL][l16][32 * k + 8 * lg]);
    const v8h al = *reinterpret_cast<const v8h *>(&L.elo[TL][l16][32 * k + 8 * lg]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      z[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(v8h, shi[u][k]), z[u], 0, 0, 0);
      z[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(v8h, slo[u][k]), z[u], 0, 0, 0);
      z[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, __builtin_bit_cast(v8h, shi[u][k]), z[u], 0, 0, 0);
    }
  }
  sign_masks<TL>(std::make_integer_sequence<int, 8>{}, z, sbits);
}
template <int BITS, int... TL>
__device__ __forceinline__ void qjl_tiles(std::integer_sequence<int, TL...>, const RoundLds<BITS> &L, int l16, int lg,
                                          const v8s (&shi)[2][4], const v8s (&slo)[2][4], uint32_t &sbits) {
  (qjl_tile<TL, BITS>(L, l16, lg, shi, slo, sbits), ...);
}

template <int DT, int BITS>
__global__ __launch_bounds__(256, 2) void encode_kernel(EncodeArgs a, int64_t num_tiles) {
  constexpr int NT = (1 << (BITS - 1)) - 1, NL = 1 << (BITS - 1);  // positive thresholds and levels
  constexpr int KP = k_page_bytes(BITS), VP = v_page_bytes(BITS), RB = k_rec_bytes(BITS);
  constexpr int KN = k_norm_off(BITS), VN = v_norm_off(BITS);
  constexpr bool kF16 = DT == TQ_F16;
  constexpr int PC = DT == TQ_F32 ? 3 : 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: no exec masking around matrix ops
  const int l16 = lane & 15, lg = lane >> 4;
  // Kernel arguments are copied to locals once: lambdas below must not
  // capture the argument struct, or it is copied to scratch memory and read
  // back through pointers.
  const int H = a.num_kv_heads;
  const void *const kin = a.k, *const vin = a.v;
  const int64_t ntok = a.num_tokens, tok_stride = a.tok_stride, head_stride = a.head_stride;
  const int64_t *const slots = a.slots;
  uint8_t *const k_cache = a.k_cache, *const v_cache = a.v_cache;
  float *const norms_out = a.norms_out;
  const int64_t nrounds = (num_tiles + kTiles - 1) / kTiles;

  __shared__ __align__(16) RoundLds<BITS> L;

  const HSets hs = make_hsets(lane, kF16 ? (uint16_t)0x3C00u : (uint16_t)0x3F80u);

  // positive thresholds and 256 x positive levels, uniform.  The levels are
  // separate scalars, chosen by selects: an array indexed by the code would
  // be moved to LDS and cost a load per coordinate.
  float tpos[NT], cp[NL];
#pragma unroll
  for (int k = 0; k < NT; ++k) tpos[k] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.t[NL + k])));
#pragma unroll
  for (int k = 0; k < NL; ++k)
    cp[k] = kResScale * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.c[NL + k])));

  // This wave's QJL rows 32w .. 32w+31 of S H as the B operand of the f16
  // MFMA, K slots in the staged residual's order: slot s <-> coordinate
  // 16 (s & 7) + (s >> 3); lane l of step k holds slots 32k + 8(l/16) .. +7.
  // The table stores exactly these registers, one 16-byte piece per lane; it
  // stays in L2 and is read again each round right before the projection, so
  // that its 64 registers are not held through the other phases.
  const uint4 *const shop = reinterpret_cast<const uint4 *>(a.SHop) + wave * 2 * 4 * 2 * 64 + lane;

  // Inputs and slot of this lane's token (l%16) in the wave's tile of round
  // R.  Every load is unconditional (past the last tile or token the address
  // repeats the last one and the result is discarded; after the wave's last
  // round every lane reads the first element, one cache line), so that the
  // number of loads in flight is known at every point and a prefetched round
  // is waited for only where it is used.
  auto load_round = [&](int64_t R, In<PC> &ik, In<PC> &iv, int64_t &slot, bool none) {
    int64_t tile = R * kTiles + wave;
    tile = tile < num_tiles ? tile : num_tiles - 1;
    const int h = (int)(tile % H);
    int64_t t = (tile / H) * kTok + l16;
    t = t < ntok ? t : ntok - 1;
    t = none ? 0 : t;
    const int64_t e0 = none ? 0 : t * tok_stride + (int64_t)h * head_stride + 8 * lg;
    // in the order of use, kept by scheduling barriers: the compiler's
    // count of loads in flight must agree at the loop entry and its back edge
    slot = slots[t];
    __builtin_amdgcn_sched_barrier(0);
    load_in<PC>(iv, vin, e0);
    __builtin_amdgcn_sched_barrier(0);
    load_in<PC>(ik, kin, e0);
    __builtin_amdgcn_sched_barrier(0);
  };

  In<PC> ik, iv;
  int64_t slot;
  load_round(blockIdx.x, ik, iv, slot, false);  // the grid has at most one workgroup per round

  for (int64_t R = blockIdx.x; R < nrounds; R += gridDim.x) {
    const int64_t tile = R * kTiles + wave;
    const bool active = tile < num_tiles;
    const int64_t t0 = (tile / H) * kTok;

    // destinations of the tile's tokens (every lane holds that of token l%16);
    // a skipped token gets a block id no other token has
    const bool ok = active && t0 + l16 < ntok && slot >= 0;
    const int blk = ok ? (int)((uint64_t)slot / kBlock) : -1 - l16;
    const int off = ok ? (int)((uint64_t)slot % kBlock) : 0;
    const bool in_order = ok && blk == __builtin_amdgcn_readlane(blk, 0) && off == l16;
    const bool full = (__ballot(in_order) & 0xFFFFull) == 0xFFFFull;  // uniform: one page, in order
    if (lane < kTok) {
      L.valid[wave][lane] = ok;
      L.blk[wave][lane] = blk;
      L.off[wave][lane] = off;
    }
    if (lane == 0) {
      L.active[wave] = active;
      L.full[wave] = full;
    }

    if (active) {
      // ---- values: C = H X^T, lane l reg i = coordinate 16m + 4(l/16) + i, token l%16
      {
        v8s xv[4][PC];
        pieces<PC>(iv, xv);
        v4f vy[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) c = mfma16<kF16>(hop(hs, k, m), xv[k][pc], c);
          vy[m] = c;
        }
        float s2 = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) s2 = fmaf(vy[m][i], vy[m][i], s2);
        s2 += xchg16(s2, lane);
        s2 += xchg32(s2, lane);
        const float sn = sqrtf(s2);  // = sqrt(128) |v|
        float T[NT];
#pragma unroll
        for (int k = 0; k < NT; ++k) T[k] = tpos[k] * sn;
        uint32_t vb[BITS];
#pragma unroll
        for (int p = 0; p < BITS; ++p) vb[p] = 0u;
        if constexpr (BITS == 3)
          value_steps(std::make_integer_sequence<int, 32>{}, vy, T[0], T[1], T[2], vb);
        else
          value_steps_b<BITS>(std::make_integer_sequence<int, 32>{}, vy, T, vb);
        // lane L = 2(4m + i) + hf holds the words of coordinates 16m + 4g + i, g = 2hf, 2hf+1
        {
          const int q = lane >> 1, hf = lane & 1, m = q >> 2, i = q & 3;
#pragma unroll
          for (int p = 0; p < BITS; ++p) {
            uint16_t *img = reinterpret_cast<uint16_t *>(L.vimg[wave] + kVPlane * p);
            img[16 * m + 4 * (2 * hf) + i] = (uint16_t)vb[p];
            img[16 * m + 4 * (2 * hf + 1) + i] = (uint16_t)(vb[p] >> 16);
          }
        }
        const float nv = sn * kInvSqrt128;
        if (lg == 0) {
          reinterpret_cast<_Float16 *>(L.vimg[wave] + VN)[l16] = to_half_sat(nv);
          L.nout[wave][l16][2] = nv;
        }
      }
      // ---- keys: C = X H, lane l reg i = token 4(l/16) + i, coordinate 16n + l%16
      {
        v8s xk[4][PC];
        pieces<PC>(ik, xk);
        v4f ky[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int pc = 0; pc < PC; ++pc) c = mfma16<kF16>(xk[k][pc], hop(hs, k, n), c);
          ky[n] = c;
        }
        float sn[4], r256[4], T[4][NT];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s2 = 0.0f;
#pragma unroll
          for (int n = 0; n < 8; ++n) s2 = fmaf(ky[n][i], ky[n][i], s2);
          s2 += xchg1(s2);
          s2 += xchg2(s2);
          s2 += xchg4(s2);
          s2 += xchg8(s2);
          sn[i] = sqrtf(s2);
          r256[i] = sn[i] > 0.0f ? kResScale / sn[i] : 0.0f;
#pragma unroll
          for (int k = 0; k < NT; ++k) T[i][k] = tpos[k] * sn[i];
        }
        uint32_t kb[BITS];
#pragma unroll
        for (int p = 0; p < BITS; ++p) kb[p] = 0u;
        float g2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float es[8][4];
        if constexpr (BITS == 3)
          key_steps(std::make_integer_sequence<int, 32>{}, ky, T, r256, cp[0], cp[1], cp[2], cp[3], kb, es, g2);
        else
          key_steps_b<BITS>(std::make_integer_sequence<int, 32>{}, ky, T, r256, cp, kb, es, g2);
        // lane L = 2(4n + i) + hf holds 16-bit pieces (coordinates 16n..+15) of tokens 4g + i, g = 2hf, 2hf+1;
        // piece n of plane p of token t is half (n & 1) of word p of record (n / 2, t)
        {
          const int q = lane >> 1, hf = lane & 1, n = q >> 2, i = q & 3;
          uint16_t *img = reinterpret_cast<uint16_t *>(L.kimg[wave]);
#pragma unroll
          for (int p = 0; p < BITS; ++p) {
            img[RB * (16 * (n >> 1) + 4 * (2 * hf) + i) / 2 + 2 * p + (n & 1)] = (uint16_t)kb[p];
            img[RB * (16 * (n >> 1) + 4 * (2 * hf + 1) + i) / 2 + 2 * p + (n & 1)] = (uint16_t)(kb[p] >> 16);
          }
        }
        // residual halves, slot 8 (l%16) + n of token 4(l/16) + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v8h hi, lo;
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            hi[n] = (_Float16)es[n][i];
            lo[n] = (_Float16)(es[n][i] - (float)hi[n]);
          }
          *reinterpret_cast<v8h *>(&L.ehi[wave][4 * lg + i][8 * l16]) = hi;
          *reinterpret_cast<v8h *>(&L.elo[wave][4 * lg + i][8 * l16]) = lo;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = g2[i];
          s += xchg1(s);
          s += xchg2(s);
          s += xchg4(s);
          s += xchg8(s);
          const float gam = sqrtf(s) * (1.0f / kResScale);
          const float nk = sn[i] * kInvSqrt128;
          const int tok = 4 * lg + i;
          if (l16 == 0) {
            reinterpret_cast<_Float16 *>(L.kimg[wave] + KN)[tok] = to_half_sat(nk);
            reinterpret_cast<_Float16 *>(L.kimg[wave] + KN + 32)[tok] = to_half_sat(gam);
            L.nout[wave][tok][0] = nk;
            L.nout[wave][tok][1] = gam;
          }
        }
      }
    }
    // this wave's projection operands (the table stays in L2), then the
    // next round's inputs (the last round repeats its own): the projection
    // waits for the former only
    v8s shi[2][4], slo[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        shi[u][k] = __builtin_bit_cast(v8s, shop[((u * 4 + k) * 2) * 64]);
        slo[u][k] = __builtin_bit_cast(v8s, shop[((u * 4 + k) * 2 + 1) * 64]);
      }
    const bool more = R + gridDim.x < nrounds;  // uniform
    load_round(more ? R + gridDim.x : R, ik, iv, slot, !more);
    lds_barrier();

    // ---- QJL projection: rows 32w .. 32w+31 for the four tiles -------------
    {
      uint32_t sbits = 0u;
      qjl_tiles(std::make_integer_sequence<int, kTiles>{}, L, l16, lg, shi, slo, sbits);
      // lane L = 2(8 tl + 4u + i) + hf: rows 16(2w+u)..+15 of tokens 4g + i, g = 2hf, 2hf+1,
      // half u of the sign word of record (w, t)
      const int q = lane >> 1, hf = lane & 1, tl = q >> 3, u = (q >> 2) & 1, i = q & 3;
      uint16_t *img = reinterpret_cast<uint16_t *>(L.kimg[tl]);
      img[RB * (16 * wave + 4 * (2 * hf) + i) / 2 + 2 * BITS + u] = (uint16_t)sbits;
      img[RB * (16 * wave + 4 * (2 * hf + 1) + i) / 2 + 2 * BITS + u] = (uint16_t)(sbits >> 16);
    }
    lds_barrier();

    // ---- write the round out --------------------------------------------------
    if (norms_out && tid < kTiles * kTok * 3) {
      const int tl = tid / (kTok * 3), n = (tid / 3) % kTok, c = tid % 3;
      const int64_t tt = R * kTiles + tl;
      const int64_t tok = (tt / H) * kTok + n;
      if (tt < num_tiles && tok < ntok) norms_out[(tok * H + tt % H) * 3 + c] = L.nout[tl][n][c];
    }
#pragma unroll
    for (int tl = 0; tl < kTiles; ++tl) {
      if (!L.active[tl]) continue;  // uniform
      const int64_t tt = R * kTiles + tl;
      const int hh = (int)(tt % H);
      if (L.full[tl]) {
        const int b0 = L.blk[tl][0];
        uint8_t *kp = k_cache + ((int64_t)b0 * H + hh) * KP;
        uint8_t *vp = v_cache + ((int64_t)b0 * H + hh) * VP;
        if (tid < KP / 16) {
          *reinterpret_cast<uint4 *>(kp + 16 * tid) = *reinterpret_cast<const uint4 *>(L.kimg[tl] + 16 * tid);
        } else if (tid < KP / 16 + VP / 16) {
          const int q = tid - KP / 16;
          *reinterpret_cast<uint4 *>(vp + 16 * q) = *reinterpret_cast<const uint4 *>(L.vimg[tl] + 16 * q);
        }
      } else {
        // token by token: K records (the four chunk records of the token,
        // RB bytes each), the scalars, and value bits merged into their pages
        // atomically
        if (tid < 4 * kTok) {
          const int n = tid >> 2, g = tid & 3;
          if (L.valid[tl][n]) {
            uint8_t *kp = k_cache + ((int64_t)L.blk[tl][n] * H + hh) * KP;
            uint8_t *dst = kp + RB * (16 * g + L.off[tl][n]);
            const uint8_t *src = L.kimg[tl] + RB * (16 * g + n);
            if constexpr (RB == 16) {
              *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
            } else {
#pragma unroll
              for (int f = 0; f < RB / 4; ++f)
                reinterpret_cast<uint32_t *>(dst)[f] = reinterpret_cast<const uint32_t *>(src)[f];
            }
          }
        } else if (tid < 5 * kTok) {
          const int n = tid - 4 * kTok;
          if (L.valid[tl][n]) {
            uint8_t *kp = k_cache + ((int64_t)L.blk[tl][n] * H + hh) * KP;
            uint8_t *vp = v_cache + ((int64_t)L.blk[tl][n] * H + hh) * VP;
            const int o = L.off[tl][n];
            *reinterpret_cast<uint16_t *>(kp + KN + 2 * o) = *reinterpret_cast<const uint16_t *>(L.kimg[tl] + KN + 2 * n);
            *reinterpret_cast<uint16_t *>(kp + KN + 32 + 2 * o) =
                *reinterpret_cast<const uint16_t *>(L.kimg[tl] + KN + 32 + 2 * n);
            *reinterpret_cast<uint16_t *>(vp + VN + 2 * o) = *reinterpret_cast<const uint16_t *>(L.vimg[tl] + VN + 2 * n);
          }
        }
        // value bits, one token at a time: wave w merges tokens w, w + 4, ..
        // of the tile; lane l owns the 32-bit word of coordinates 2l, 2l + 1
        // of each plane (16-bit words, token o of the page at bit o), so a
        // token is two coalesced 256-byte atomics per plane.  Tokens that share
        // a page touch different bits of the same words: the atomics keep them
        // apart, in this call and across the waves of the grid.
        for (int n = wave; n < kTok; n += 4) {  // uniform
          if (!__builtin_amdgcn_readfirstlane((int)L.valid[tl][n])) continue;  // uniform
          const int bn = __builtin_amdgcn_readfirstlane(L.blk[tl][n]);
          const int o = __builtin_amdgcn_readfirstlane(L.off[tl][n]);
          uint8_t *vp = v_cache + ((int64_t)bn * H + hh) * VP;
#pragma unroll
          for (int p = 0; p < BITS; ++p) {
            const uint32_t w2 = reinterpret_cast<const uint32_t *>(L.vimg[tl] + kVPlane * p)[lane];
            const uint32_t b = ((w2 >> n) & 1u) | (((w2 >> (16 + n)) & 1u) << 16);
            const uint32_t set = b << o, clr = (0x10001u << o) & ~set;
            // global (not flat) atomics: a pending flat operation would make
            // every later wait on the memory counters wait for all of them
            gword *w32 = reinterpret_cast<gword *>(reinterpret_cast<uintptr_t>(vp + kVPlane * p + 4 * lane));
            __hip_atomic_fetch_and(w32, ~clr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(w32, set, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        // the stores in the loops above leave an unbounded count of memory
        // operations in flight for the compiler, which would then wait for all
        // of them (the next round's inputs included) at the next use of a
        // load: wait here, on this path only
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
    }
    lds_barrier();  // the round's LDS state is rewritten by the next round
  }
}

template <int DT>
hipError_t launch_append(const EncodeArgs &a, hipStream_t stream) {
  const int64_t waves = a.num_tokens * a.num_kv_heads;
  const dim3 grid((unsigned)((waves + kAppendWaves - 1) / kAppendWaves));
  switch (a.cb.bits) {
    case 2: hipLaunchKernelGGL((append_kernel<DT, 2>), grid, dim3(64 * kAppendWaves), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((append_kernel<DT, 3>), grid, dim3(64 * kAppendWaves), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((append_kernel<DT, 4>), grid, dim3(64 * kAppendWaves), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const EncodeArgs &a, int64_t tiles, hipStream_t stream) {
  const int64_t rounds = (tiles + kTiles - 1) / kTiles;
  const int64_t grid = rounds < 512 ? rounds : 512;  // persistent: two workgroups per CU
  switch (a.cb.bits) {
    case 2: hipLaunchKernelGGL((encode_kernel<DT, 2>), dim3((unsigned)grid), dim3(256), 0, stream, a, tiles); break;
    case 3: hipLaunchKernelGGL((encode_kernel<DT, 3>), dim3((unsigned)grid), dim3(256), 0, stream, a, tiles); break;
    case 4: hipLaunchKernelGGL((encode_kernel<DT, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a, tiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream) {
  const int64_t groups = (a.num_tokens + kTok - 1) / kTok;
  const int64_t tiles = groups * a.num_kv_heads;
  if (a.num_tokens * a.num_kv_heads <= kAppendMaxVectors) {  // a few vectors: one wave each
    switch (a.dtype) {
      case TQ_BF16: return launch_append<TQ_BF16>(a, stream);
      case TQ_F16: return launch_append<TQ_F16>(a, stream);
      case TQ_F32: return launch_append<TQ_F32>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.dtype) {
    case TQ_BF16: return launch_dt<TQ_BF16>(a, tiles, stream);
    case TQ_F16: return launch_dt<TQ_F16>(a, tiles, stream);
    case TQ_F32: return launch_dt<TQ_F32>(a, tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
