// Device helpers shared by the encode and attention kernels (wave64 gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

constexpr float kInvSqrt128 = 0.08838834764831845f;

// Workgroup barrier that orders LDS only.  __syncthreads() also makes every
// outstanding global store visible first (a full vmcnt wait); kernels whose
// barriers guard nothing but LDS use this one and keep stores in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A context length above the planned maximum breaks the caller contract; it
// is cut to what the block table row and the split plan cover, so that no
// access leaves the block table or the partials.
__device__ __forceinline__ int clamped_context(const DecodeArgs &a, int b) {
  return min(max(a.context_lens[b], 0), a.ctx_cap);
}

// Sliding window over a rotating cache: the first page-aligned position any
// query of the call can see (the oldest key of its first query, rounded down
// to its page); every pass walks sequence b's keys from there to its end.
// Without a window the walk starts at 0.
__device__ __forceinline__ int seq_base(const DecodeArgs &a, int L) {
  return a.window > 0 ? (max(0, L - a.q_len - a.window + 1) & ~15) : 0;
}
// Block-table entry of logical page P: with a window the row is a ring of
// max_blocks pages, so position p sits in entry (p / 16) mod max_blocks.
__device__ __forceinline__ int page_entry(const DecodeArgs &a, int P) {
  return a.window > 0 ? (int)((unsigned)P % (unsigned)a.max_blocks) : P;
}
// Lower end (inclusive) of the keys a query sees, given its exclusive upper
// end `lim`: lim - window with a window, else none.
__device__ __forceinline__ int window_low(const DecodeArgs &a, int lim) {
  return a.window > 0 ? lim - a.window : INT_MIN;
}

__device__ __forceinline__ float load_as_float(const void *p, int dtype, int64_t i) {
  if (dtype == TQ_F32) return static_cast<const float *>(p)[i];
  if (dtype == TQ_F16) return (float)static_cast<const _Float16 *>(p)[i];
  const uint32_t bits = static_cast<const uint16_t *>(p)[i];
  return __uint_as_float(bits << 16);
}

__device__ __forceinline__ void store_from_float(void *p, int dtype, int64_t i, float v) {
  if (dtype == TQ_F32) {
    static_cast<float *>(p)[i] = v;
  } else if (dtype == TQ_F16) {
    static_cast<_Float16 *>(p)[i] = (_Float16)v;
  } else {
    // round to nearest even bf16 (NaN kept quiet)
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      u |= 0x00400000u;
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);
    }
    static_cast<uint16_t *>(p)[i] = (uint16_t)(u >> 16);
  }
}

// ---- lane exchanges: value held by lane (lane ^ s), all in VALU ----------------
// strides 1, 2: DPP quad_perm; 4: row_half_mirror then quad_perm [3,2,1,0]
// (lane ^ 7 ^ 3); 8: row_ror:8 inside a 16-lane row; 16 and 32: the gfx950
// permlane16/permlane32 swaps (each returns both halves; the lane keeps the
// one that came from the other row / half).
__device__ __forceinline__ float xchg1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float xchg2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float xchg4(float x) {
  const int m = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false);
  return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false));
}
__device__ __forceinline__ float xchg8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float xchg16(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float xchg32(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(((lane >> 5) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float xchg(float x, int s, int lane) {
  switch (s) {
    case 1: return xchg1(x);
    case 2: return xchg2(x);
    case 4: return xchg4(x);
    case 8: return xchg8(x);
    case 16: return xchg16(x, lane);
    default: return xchg32(x, lane);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o <= 32; o <<= 1) v += xchg(v, o, lane);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o <= 32; o <<= 1) v = fmaxf(v, xchg(v, o, lane));
  return v;
}

// Orthonormal Walsh-Hadamard transform of 128 values held two per lane
// (lane l holds coordinates l and l + 64), Sylvester order: the stride-64
// butterfly is inside the lane, strides 32..1 pair lane l with lane l ^ s.
// (lilting.ch article, "Walsh-Hadamard Transform（WHT）の役割": an orthogonal,
// add/sub-only, divide-and-conquer rotation.)
__device__ __forceinline__ void wave_fwht128(float &r0, float &r1, int lane) {
  const float a = r0 + r1, b = r0 - r1;
  r0 = a;
  r1 = b;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float p0 = xchg(r0, s, lane), p1 = xchg(r1, s, lane);
    const bool upper = (lane & s) != 0;
    r0 = upper ? (p0 - r0) : (r0 + p0);
    r1 = upper ? (p1 - r1) : (r1 + p1);
  }
  r0 *= kInvSqrt128;
  r1 *= kInvSqrt128;
}

// Sum over the wave, returned in every lane: inclusive scans inside each
// 16-lane row (DPP row_shr 1, 2, 4, 8; out-of-row sources read 0), then
// row_bcast:15 and row_bcast:31 carry the row totals up to lane 63, which is
// read back as a uniform value.
__device__ __forceinline__ float wave_sum_u(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

// Walsh-Hadamard transform (unnormalised, Sylvester order) of 128 values held
// two per lane, lane l starting with coordinates l (in a) and l + 64 (in b).
// The stride-64 butterfly is in-lane; permlane32_swap then regroups so that
// lane m < 32 holds (m, m+32) and lane 32+m holds (64+m, 96+m), making the
// stride-32 butterfly in-lane; permlane16_swap regroups again so that lane
// 16r+i holds (32r+i, 32r+16+i) for stride 16.  Strides 8..1 stay inside
// 16-lane rows (DPP).  On return lane 16r+i holds coordinate 32r+i in a and
// 32r+16+i in b.
__device__ __forceinline__ void fwht128_regroup(float &a, float &b, int lane) {
  float s = a + b, d = a - b;
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(d), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
  s = a + b;
  d = a - b;
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(d), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
  s = a + b;
  d = a - b;
  a = s;
  b = d;
#pragma unroll
  for (int st = 8; st >= 1; st >>= 1) {
    const float sg = (lane & st) ? -1.0f : 1.0f;
    const float pa = xchg(a, st, lane), pb = xchg(b, st, lane);
    a = fmaf(sg, a, pa);
    b = fmaf(sg, b, pb);
  }
}

// Coordinates held by lane l after fwht128_regroup.
__device__ __forceinline__ int regroup_coord_a(int lane) { return 32 * (lane >> 4) + (lane & 15); }
__device__ __forceinline__ int regroup_coord_b(int lane) { return 32 * (lane >> 4) + 16 + (lane & 15); }

// 32-bit word r (coordinates 32r .. 32r+31) of a 128-bit plane record from
// the ballots of the a and b halves in the regrouped layout.
__device__ __forceinline__ uint32_t regroup_plane_word(uint64_t ma, uint64_t mb, int r) {
  return (uint32_t)((ma >> (16 * r)) & 0xFFFFull) | ((uint32_t)((mb >> (16 * r)) & 0xFFFFull) << 16);
}

// Level index of y: the number of thresholds strictly below y (a value on a
// threshold goes to the lower cell), compared in fp32.
__device__ __forceinline__ int cell_index(float y, const Codebook &cb) {
  int idx = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) idx += (cb.t[j] < y) ? 1 : 0;
  return idx;
}

__device__ __forceinline__ _Float16 to_half_sat(float v) {
  return (_Float16)fminf(v, 65504.0f);
}

// A matrix instruction writes its whole result, on every lane, whatever the
// exec mask.  The compiler may nevertheless move one into a branch taken by
// the lanes that use its result (a score formed only where the mask keeps
// it): the lanes outside the branch then find their own value in the result
// registers overwritten (a masked -inf replaced by a finite score).  Pinning
// the result in registers right after the chain that forms it keeps the
// instructions out of any such branch.
template <class V>
__device__ __forceinline__ void pin_result(V &x) {
  asm volatile("" : "+v"(x));
}

}  // namespace tq
