// Device helpers shared by the encode and attention kernels (wave64 gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

constexpr float kInvSqrt128 = 0.08838834764831845f;

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
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
    const float p0 = __shfl_xor(r0, s), p1 = __shfl_xor(r1, s);
    const bool upper = (lane & s) != 0;
    r0 = upper ? (p0 - r0) : (r0 + p0);
    r1 = upper ? (p1 - r1) : (r1 + p1);
  }
  r0 *= kInvSqrt128;
  r1 *= kInvSqrt128;
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

}  // namespace tq
