// Matrix-core helpers for attention over bit-plane pages (gfx950).
//
// The scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 (fp32 accumulate, E8M0
// scales) is used with:
//   B = fp4 e2m1 values read straight from packed bits: one and_or per 8
//       values;
//   A = a float operand written as integer digits, one digit per A row, each
//       row's place value carried by its scale, as fp6 e2m3 codes: the code
//       of d/8 is sign << 5 | |d| for |d| <= 16, and the instruction runs at
//       the fp4/fp6 rate (about 1.8x the fp8 x fp4 rate, measured).
// Operand layouts (lane l, measured on gfx950 with one-hot operands):
//   A fp6: row l%16; its 32 six-bit codes, packed in order (code s at bits
//      6s .. 6s+5 of registers 0..5), hold logical K 32*(l/16) + s;
//   B fp4: column l%16; its 32 nibbles (4 registers) hold logical K
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

// Coordinate (token) that logical K index kap of a B operand made by b_split
// from the 32-bit word of coordinates 32*(kap/32) .. +31 stands for: nibble
// t of register v holds bit 4t + v.
__device__ __forceinline__ int b_coord(int kap) { return 32 * (kap >> 5) + 4 * (kap & 7) + ((kap >> 3) & 3); }

// B operand from 32 bits with one instruction per register, avoiding fp4
// subnormals: register v keeps bit v of each nibble in place, giving the e2m1
// values alpha_v + beta_v * bit:
//   v = 0: nibble 0x6 | bit0 -> 4.0 or 6.0   (alpha 4, beta 2)
//   v = 1: nibble 0x4 | bit1 -> 2.0 or 4.0   (alpha 2, beta 2)
//   v = 2: nibble bit2       -> 0 or 2.0     (alpha 0, beta 2)
//   v = 3: nibble 0x2 | bit3 -> 1.0 or -1.0  (alpha 1, beta -2)
// A contraction against the +-1 values 1 - 2 bit is recovered by scaling the
// A value of a K slot in register v by f_v = -2/beta_v (-1, -1, -1, +1: no
// digit grows, so fp6 digits stay exact) and adding sum_k A_k (1 - f_v
// alpha_v), i.e. weights 5, 3, 1, 0:
//   sum_k A_k (1 - 2 b_k) = sum_k (f_v A_k) B'_k + sum_k (1 - f_v alpha_v) A_k.
__device__ __forceinline__ v8i b_split(uint32_t P) {
  v8i b;
  b[0] = (int)((P & 0x11111111u) | 0x66666666u);
  b[1] = (int)((P & 0x22222222u) | 0x44444444u);
  b[2] = (int)(P & 0x44444444u);
  b[3] = (int)((P & 0x88888888u) | 0x22222222u);
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}
// Register of logical K index kap inside its 32-wide block and the A factor
// that goes with b_split.
__device__ __forceinline__ int b_reg(int kap) { return (kap >> 3) & 3; }
__device__ __forceinline__ float b_split_factor(int kap) { return b_reg(kap) == 3 ? 1.0f : -1.0f; }

// A fp6 e2m3 (registers 0..5), B fp4.
__device__ __forceinline__ v4f mfma_f6f4(const v8i &A, const v8i &B, const v4f &C, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, 2, 4, 0, scale_a, 0, kE8M0One);
}
constexpr int kFp6Exp = 3;  // fp6 digit codes stand for d / 8

}  // namespace tq
