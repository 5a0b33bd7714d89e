// One-wave-per-vector encoder for small appends, shared by the encode call
// and the fused decode step (SwiftLM README, "TurboQuantization: KV Cache
// Compression": K-cache steps 1-5 and the V-cache paragraph).
#pragma once

#include "tq_common.hpp"

namespace tq {
namespace {

// ---- small appends: one wave per (token, KV head) ---------------------------
// A decode step appends one token per sequence: a few hundred vectors that
// fill few 16-token tiles, so the tiled kernel above runs on one or two
// workgroups and its whole chain of latencies is the call's time.  Here
// every vector has a wave of its own: lane l holds coordinates l and l + 64;
// the rotation is the butterfly in registers, the codes come from per-lane
// compares (count c of the positive thresholds below |y|, rank 2^(B-1) + c or
// 2^(B-1) - 1 - c) and wave ballots give the bit-planes; the QJL projection
// z = S r (r = H e, the residual back in the original domain) takes row l and
// row l + 64 per lane from S^T (coalesced) against r broadcast from LDS, in
// fp32.  The record goes out as the token's chunk records, its scalars, and
// the value bits merged with two atomics per plane word, so tokens that share
// a page (and calls of the tiled kernel) never overwrite each other.
// kAppendWaves such vectors share a workgroup.
typedef __attribute__((address_space(1))) uint32_t append_gword;

template <int DT>
__device__ __forceinline__ float load_elem(const void *p, int64_t i) {
  if constexpr (DT == TQ_F32) return static_cast<const float *>(p)[i];
  if constexpr (DT == TQ_F16) return (float)static_cast<const _Float16 *>(p)[i];
  return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
}

// Workgroup `wg` of an append launch (kAppendWaves waves, one vector each;
// rsh: kAppendWaves x 128 floats of LDS).  Waves past the last vector, or of a
// skipped token, return at once (no workgroup barrier follows).
template <int DT, int BITS>
__device__ __attribute__((always_inline)) void append_body(const EncodeArgs &a, float (*rsh)[kHeadDim], int64_t wg) {
  constexpr int NT = (1 << (BITS - 1)) - 1, NL = 1 << (BITS - 1);
  constexpr int KP = k_page_bytes(BITS), VP = v_page_bytes(BITS), RB = k_rec_bytes(BITS);
  constexpr int KN = k_norm_off(BITS), VN = v_norm_off(BITS);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t pair = wg * kAppendWaves + wave;
  const int H = a.num_kv_heads;
  if (pair >= a.num_tokens * H) return;  // uniform per wave (no block barrier below)
  const int64_t t = pair / H;
  const int h = (int)(pair % H);
  const int64_t slot = a.slots[t];
  if (slot < 0) return;  // uniform: a skipped token
  const int64_t blk = slot / kBlock;
  const int off = (int)(slot % kBlock);
  const int64_t e0 = t * a.tok_stride + (int64_t)h * a.head_stride;
  float tpos[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) tpos[k] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.t[NL + k])));
  // the positive levels, read where they are selected (kept out of an array:
  // a select between two array elements would become an indexed load from
  // private memory)
  auto level = [&](int k) __attribute__((always_inline)) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.c[NL + k])));
  };

  // codes of one rotated vector (lane: coordinates l, l + 64): rank bits as
  // per-plane ballots, the u-domain residual, and the norm
  auto quantise = [&](float x0, float x1, uint64_t (&pl)[BITS][2], float (&e)[2], float &n)
      __attribute__((always_inline)) {
    n = sqrtf(wave_sum(fmaf(x0, x0, x1 * x1)));
    float y[2] = {x0, x1};
    wave_fwht128(y[0], y[1], lane);
    const float rinv = n > 0.0f ? 1.0f / n : 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float ay = fabsf(y[j]);
      int cnt = 0;
      float lv = level(0);
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        const bool above = ay > tpos[k] * n;
        cnt += above ? 1 : 0;
        lv = above ? level(k + 1) : lv;
      }
      const bool pos = y[j] > 0.0f;
      const int rank = pos ? NL + cnt : NL - 1 - cnt;
      e[j] = fmaf(y[j], rinv, pos ? -lv : lv);
#pragma unroll
      for (int p = 0; p < BITS; ++p) pl[p][j] = __ballot((rank >> p) & 1);
    }
  };

  uint8_t *const kp = a.k_cache + (blk * H + h) * KP;
  uint8_t *const vp = a.v_cache + (blk * H + h) * VP;
  // both inputs are requested before any work, then the first half of the
  // projection's S^T columns (rows l, l + 64 for k < 64), which do not depend
  // on the vector
  const float xv0 = load_elem<DT>(a.v, e0 + lane), xv1 = load_elem<DT>(a.v, e0 + 64 + lane);
  const float xk0 = load_elem<DT>(a.k, e0 + lane), xk1 = load_elem<DT>(a.k, e0 + 64 + lane);
  const float *st = a.St;
  float sa[64], sb[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    sa[i] = st[i * kQjlDim + lane];
    sb[i] = st[i * kQjlDim + 64 + lane];
  }

  // ---- value -------------------------------------------------------------
  {
    const float x0 = xv0, x1 = xv1;
    uint64_t pl[BITS][2];
    float e[2], n;
    quantise(x0, x1, pl, e, n);
    // lane l owns the 32-bit word of coordinates 2l, 2l + 1 of each plane
    const int c = 2 * lane, half = c >> 6, sh = c & 63;
    append_gword *w32base = reinterpret_cast<append_gword *>(reinterpret_cast<uintptr_t>(vp + 4 * lane));
#pragma unroll
    for (int p = 0; p < BITS; ++p) {
      const uint64_t m = pl[p][half];
      const uint32_t b = (uint32_t)((m >> sh) & 1u) | ((uint32_t)((m >> (sh + 1)) & 1u) << 16);
      const uint32_t set = b << off, clr = (0x10001u << off) & ~set;
      append_gword *w32 = w32base + (kVPlane / 4) * p;
      __hip_atomic_fetch_and(w32, ~clr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(w32, set, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) reinterpret_cast<_Float16 *>(vp + VN)[off] = to_half_sat(n);
    if (a.norms_out && lane == 0) a.norms_out[(t * H + h) * 3 + 2] = n;
  }
  // ---- key ---------------------------------------------------------------
  {
    const float x0 = xk0, x1 = xk1;
    uint64_t pl[BITS][2];
    float e[2], n;
    quantise(x0, x1, pl, e, n);
    const float gam = sqrtf(wave_sum(fmaf(e[0], e[0], e[1] * e[1])));
    // z = S r, r = H e: rows l and l + 64 against r from LDS
    float r0 = e[0], r1 = e[1];
    wave_fwht128(r0, r1, lane);
    rsh[wave][lane] = r0;
    rsh[wave][lane + 64] = r1;
    __builtin_amdgcn_wave_barrier();
    float z0 = 0.0f, z1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kHeadDim; kb += 64) {  // k < 64 from the registers loaded first
      if (kb > 0) {
#pragma unroll
        for (int i = 0; i < 64; ++i) {
          sa[i] = st[(kb + i) * kQjlDim + lane];
          sb[i] = st[(kb + i) * kQjlDim + 64 + lane];
        }
      }
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        const float4 r4 = *reinterpret_cast<const float4 *>(&rsh[wave][kb + i]);
        z0 = fmaf(sa[i], r4.x, z0);
        z1 = fmaf(sb[i], r4.x, z1);
        z0 = fmaf(sa[i + 1], r4.y, z0);
        z1 = fmaf(sb[i + 1], r4.y, z1);
        z0 = fmaf(sa[i + 2], r4.z, z0);
        z1 = fmaf(sb[i + 2], r4.z, z1);
        z0 = fmaf(sa[i + 3], r4.w, z0);
        z1 = fmaf(sb[i + 3], r4.w, z1);
      }
    }
    const uint64_t s0 = __ballot(z0 >= 0.0f), s1 = __ballot(z1 >= 0.0f);
    // the token's record words: lane j < 4 (BITS + 1) writes field j % (BITS + 1)
    // of chunk j / (BITS + 1) (chunks 0, 1 from the low masks, 2, 3 the high)
    if (lane < 4 * (BITS + 1)) {
      const int g = lane / (BITS + 1), f = lane % (BITS + 1);
      uint64_t m = 0;
#pragma unroll
      for (int p = 0; p < BITS; ++p) m = f == p ? pl[p][g >> 1] : m;
      m = f == BITS ? (g < 2 ? s0 : s1) : m;
      const uint32_t w = (uint32_t)(m >> (32 * (g & 1)));
      *reinterpret_cast<uint32_t *>(kp + RB * (16 * g + off) + 4 * f) = w;
    }
    if (lane == 0) {
      reinterpret_cast<_Float16 *>(kp + KN)[off] = to_half_sat(n);
      reinterpret_cast<_Float16 *>(kp + KN + 32)[off] = to_half_sat(gam);
      if (a.norms_out) {
        a.norms_out[(t * H + h) * 3 + 0] = n;
        a.norms_out[(t * H + h) * 3 + 1] = gam;
      }
    }
  }
}

template <int DT, int BITS>
__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(EncodeArgs a) {
  __shared__ __align__(16) float rsh[kAppendWaves][kHeadDim];
  append_body<DT, BITS>(a, rsh, blockIdx.x);
}

}  // namespace
}  // namespace tq
