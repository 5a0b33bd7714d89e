// Matrix-core helpers for attention over bit-plane pages (gfx950).
//
// The scaled fp8 x fp4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, A = fp8 e4m3,
// B = fp4 e2m1, fp32 accumulate, E8M0 scales) is used with:
//   B = +-1 values read straight from packed bits: one and_or per 8 values;
//   A = a float operand written as integer digits (exact in e4m3), one digit
//       per A row, each row's place value carried by its scale.
// Operand layouts (lane l, measured on gfx950 with one-hot operands):
//   A: row l%16; its 32 bytes (8 registers) hold logical K
//      64*(s/16) + 16*(l/16) + s%16 for byte s = 0..31;
//   B: column l%16; its 32 nibbles (4 registers) hold logical K
//      32*(l/16) + s for nibble s = 0..31;
//   C: register i holds row 4*(l/16)+i, column l%16;
//   A scale of lane l: row l%16, logical K 32*(l/16) .. +31 (one per row and
//   32-wide K block); B scale of lane l likewise for column l%16.
#pragma once

#include "tq_common.hpp"

namespace tq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kE8M0One = 127;  // E8M0 encoding of 2^0

// Logical K of A byte s in lane group ga.
__device__ __forceinline__ int mfma_a_slot_k(int ga, int s) { return 64 * (s >> 4) + 16 * ga + (s & 15); }

// Coordinate (token) that logical K index kap of a B operand made by b_pm1
// from the 32-bit word of coordinates 32*(kap/32) .. +31 stands for: nibble
// t of register v holds bit 4t + v.
__device__ __forceinline__ int b_coord(int kap) { return 32 * (kap >> 5) + 4 * (kap & 7) + ((kap >> 3) & 3); }
// Inverse within a 32-wide block: logical K of coordinate 32a + 4t + v.
__device__ __forceinline__ int b_kappa(int c) { return 32 * (c >> 5) + 8 * (c & 3) + ((c & 31) >> 2); }

// B operand of 32 values +-1 from 32 bits: value = 1 - 2 * bit.  Register v,
// nibble t takes bit 4t + v (shifted to the fp4 sign position, magnitude 1.0).
__device__ __forceinline__ v8i b_pm1(uint32_t P) {
  v8i b;
  b[0] = (int)(((P << 3) & 0x88888888u) | 0x22222222u);
  b[1] = (int)(((P << 2) & 0x88888888u) | 0x22222222u);
  b[2] = (int)(((P << 1) & 0x88888888u) | 0x22222222u);
  b[3] = (int)((P & 0x88888888u) | 0x22222222u);
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

__device__ __forceinline__ v4f mfma_f8f4(const v8i &A, const v8i &B, const v4f &C, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, 0, 4, 0, scale_a, 0, kE8M0One);
}

}  // namespace tq
