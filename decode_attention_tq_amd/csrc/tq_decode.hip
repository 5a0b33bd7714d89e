// Attention read directly from the compressed, paged cache (gfx950).
//
// Launches on the caller's stream:
//   1. query prep  : per query row, q' = H q (rotated once) and
//                    s = sqrt(pi/2)/m * S q (the QJL side of the score), so
//                    no split repeats them;
//   2. split pass  : one workgroup per (sequence and query position, KV head,
//                    token chunk); scores every key of its chunk against the G
//                    grouped query heads from the packed bit-planes,
//                        score = scale * n_k * (<q', c[idx]> + gamma <s, sigma>),
//                    keeps an online softmax and accumulates values in the
//                    rotated domain, acc' += p * n_v * c[idx_v];
//   3. merge       : log-sum-exp combine of the chunks, o' = acc'/l, and one
//                    inverse FWHT per output row (o = H o', H = H^T = H^-1).
// The score is the QJL-corrected inner-product estimate for the key record of
// the SwiftLM README ("TurboQuantization", K-cache step 5) evaluated in the
// rotated domain: <q, H^T c> = <H q, c>.

#include <math.h>
#include <stddef.h>

#include <mutex>
#include <type_traits>

#include "tq_mfma.hpp"
#include "tq_append.hpp"

namespace tq {
namespace {

constexpr int kPartStride = 132;  // m (log2 units), l, pad, pad, acc[128]
constexpr float kLog2e = 1.4426950408889634f;

// ---- balanced plan of the matrix-core decode pass ----------------------------
// Sequence s has T_s = ceil(L_s / 128) tiles; each of its Hkv groups is cut
// into k_s = ceil(T_s / per) ranges of per tiles, one workgroup each, and the
// ranges are numbered densely, sequence-major then head-major.  per is the
// smallest multiple of 4 in [bal_min, 64] (the four waves of a workgroup
// then get equal tiles) whose ranges number at most bal_target (the count
// that fills the compute units once), or 64; a caller's fixed bal_per
// overrides it.  Every wave of a workgroup (and of the merge and
// window passes) computes the same values from the context lengths, 64
// sequences at a time.
// Inclusive prefix sum over the wave: scans inside each 16-lane row (DPP
// row_shr 1, 2, 4, 8; out-of-row sources read 0), then row_bcast:15 and
// row_bcast:31 carry the row totals up.
__device__ __forceinline__ int wave_incl_scan_int(int x, int lane) {
  (void)lane;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}
// ceil(T / p) for 0 <= T < 2^24 and 1 <= p <= 64, from a float estimate of
// the quotient (within 2 of the true one) corrected in two steps either way.
__device__ __forceinline__ int ceil_div_small(int T, int p, float rp) {
  int q = (int)((float)T * rp);
  int r = T - q * p;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (r < 0) { --q; r += p; }
    if (r >= p) { ++q; r -= p; }
  }
  return q + (r > 0 ? 1 : 0);
}
__device__ __forceinline__ int seq_tiles(const DecodeArgs &a, int s) {
  if (s >= a.num_seqs) return 0;
  const int L = clamped_context(a, s);
  return (L - seq_base(a, L) + 127) >> 7;
}
// The tile counts of sequences c0 + lane: for up to 64 sequences they are
// read once (t0, loaded by the caller at its start) and every later step
// works in registers; larger batches read them again per block of 64.
__device__ __forceinline__ int block_tiles(const DecodeArgs &a, int t0, int c0, int lane) {
  return a.num_seqs <= 64 ? t0 : seq_tiles(a, c0 + lane);
}
// Ranges of all groups for a range length of p tiles.
__device__ __forceinline__ int bal_ranges(const DecodeArgs &a, int t0, int p) {
  const int lane = threadIdx.x & 63;
  int tot = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64)  // uniform
    tot += __builtin_amdgcn_readlane(wave_incl_scan_int((block_tiles(a, t0, c0, lane) + p - 1) / p, lane), 63);
  return tot * a.num_kv_heads;
}
__device__ __forceinline__ int bal_per(const DecodeArgs &a, int t0) {
  if (a.bal_per > 0) return a.bal_per;
  if (a.num_seqs <= 64) {
    // lane = sequence: try p = 4, 8, ... in turn (a short chain: the
    // filling count is usually met within a few steps)
    const int lane = threadIdx.x & 63;
    for (int p = max(4, (a.bal_min + 3) & ~3); p < 64; p += 4) {  // uniform
      const int k = (t0 + p - 1) / p;  // t0 = 0 past the last sequence
      const int tot = __builtin_amdgcn_readlane(wave_incl_scan_int(k, lane), 63);
      if (tot * a.num_kv_heads <= a.bal_target) return p;
    }
    return 64;
  }
  int lo = (a.bal_min + 3) >> 2, hi = 16;  // p = 4 m
  while (lo < hi) {  // uniform
    const int mid = (lo + hi) >> 1;
    if (bal_ranges(a, t0, 4 * mid) <= a.bal_target) hi = mid; else lo = mid + 1;
  }
  return 4 * lo;
}
// Workgroup w's range: sequence b, KV head h, range index j of the group
// and the group's tile count; b = num_seqs when w is past the last range.
__device__ __forceinline__ void bal_locate(const DecodeArgs &a, int t0, int per, int w, int &b, int &h, int &j,
                                           int &Tb) {
  const int lane = threadIdx.x & 63, H = a.num_kv_heads;
  int base = 0;
  b = a.num_seqs;
  h = j = Tb = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {  // uniform
    const int T = block_tiles(a, t0, c0, lane);
    const int k = (T + per - 1) / per;
    const int incl = wave_incl_scan_int(H * k, lane);
    const int ctot = __builtin_amdgcn_readlane(incl, 63);
    if (w < base + ctot) {  // uniform: w lies in this block of sequences
      // sequences whose ranges end at or before w (empty ones included) come first
      const int i = __builtin_amdgcn_readfirstlane(__popcll(__ballot(base + incl <= w)));
      b = c0 + i;
      Tb = __builtin_amdgcn_readlane(T, i);
      const int kb = __builtin_amdgcn_readlane(k, i);
      const int off = w - (base + __builtin_amdgcn_readlane(incl, i) - H * kb);
      h = off / kb;
      j = off - h * kb;
      return;
    }
    base += ctot;
  }
}

// ---- 1. query prep (vector and prefill passes): a workgroup per query row -----
// Grid (sequence x position x KV head, head of the group).  Thread (i, half)
// forms half of (S q)_i from S[i][64*half .. +64) held in registers; wave 0
// rotates q.  The matrix-core split pass forms its operands itself (below).
__device__ __forceinline__ int bound_exponent(float M) {  // M < 2^E for finite M > 0
  const int ex = (int)((__float_as_uint(M) >> 23) & 0xFFu);
  return ex == 0 ? -126 : ex - 126;
}

__global__ __launch_bounds__(256) void query_prep_kernel(DecodeArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group;
  const int64_t grp = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t row = grp * G + g;
  __shared__ __align__(16) float qs[kHeadDim];
  __shared__ float part[2][kQjlDim];
  __shared__ float qp[256];
  if (tid < kHeadDim) qs[tid] = load_as_float(a.q, a.q_dtype, row * kHeadDim + tid);
  // thread (i, half): half of (S q)_i from S[i][64 half .. +64), read from
  // S^T so that a wave's loads are 256 contiguous bytes; four independent sums
  const int i = tid & 127, half = tid >> 7;
  float sk[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) sk[k] = a.St[(half * 64 + k) * kQjlDim + i];
  lds_barrier();
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const float4 *q4 = reinterpret_cast<const float4 *>(qs + 64 * half);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float4 x = q4[k];  // the same address in every lane: a broadcast
    acc[0] = fmaf(sk[4 * k], x.x, acc[0]);
    acc[1] = fmaf(sk[4 * k + 1], x.y, acc[1]);
    acc[2] = fmaf(sk[4 * k + 2], x.z, acc[2]);
    acc[3] = fmaf(sk[4 * k + 3], x.w, acc[3]);
  }
  part[half][i] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (wave == 0) {
    float x0 = qs[lane], x1 = qs[lane + 64];
    wave_fwht128(x0, x1, lane);
    qp[lane] = x0;
    qp[lane + 64] = x1;
  }
  lds_barrier();
  if (tid < kQjlDim) qp[128 + tid] = a.cb.qjl_scale * (part[0][tid] + part[1][tid]);
  lds_barrier();
  a.qprep[row * 256 + tid] = qp[tid];
}

// ---- 2. split pass (vector ALU) --------------------------------------------
// G is the capacity (1, 2, 4, 8 or 16 heads); the call's group size
// (a.group <= G) indexes the rows, the heads past it score zero queries and
// write nothing.  BITS: code width of the pages (2, 3 or 4).
template <int G, int BITS>
__global__ __launch_bounds__(256) void split_valu_kernel(DecodeArgs a) {
  constexpr int NL = 1 << BITS;  // levels
  constexpr int KP = k_page_bytes(BITS), VP = v_page_bytes(BITS), RB = k_rec_bytes(BITS);
  const int Gr = a.group;
  const int bt = blockIdx.x;  // b * q_len + t
  const int h = blockIdx.y;
  const int split = blockIdx.z;
  const int b = bt / a.q_len, t = bt % a.q_len;
  const int L = clamped_context(a, b);
  const int vis = max(0, L - a.q_len + t + 1);
  const int lo = window_low(a, vis);  // keys before lo are outside the window
  const int s0 = seq_base(a, L) + split * a.split_tokens;
  const int s1 = min(s0 + a.split_tokens, vis);
  if (s0 >= s1) return;  // uniform: this chunk holds no visible key
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // main loop: qp[G][128] | sq[G][128] | pn[4][G][64]; after it: red[4][G][128]
  __shared__ float smem[G * 512];
  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ float lut[NL];
  float *qp = smem;
  float *sq = smem + G * 128;
  float *pn = smem + G * 256;

  const int64_t row0 = (int64_t)bt * a.num_q_heads + (int64_t)h * Gr;
  for (int idx = tid; idx < G * 256; idx += 256) {
    const int g = idx >> 8, c = idx & 255;
    const float v = g < Gr ? a.qprep[(row0 + g) * 256 + c] : 0.0f;
    if (c < 128) qp[g * 128 + c] = v; else sq[g * 128 + c - 128] = v;
  }
  if (tid < NL) {
    // read the levels into registers first: a select over kernel-argument
    // fields can be folded into a lane-indexed memory load
    float cv[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) cv[j] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.c[j])));
    float c = cv[0];
#pragma unroll
    for (int j = 1; j < NL; ++j) c = (tid == j) ? cv[j] : c;
    lut[tid] = c;
  }
  lds_barrier();

  const int32_t *btab = a.block_tables + (int64_t)b * a.max_blocks;
  const float cs = a.scale * kLog2e;  // scores in log2 units
  float m[G], l[G], acc0[G], acc1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    acc0[g] = 0.0f;
    acc1[g] = 0.0f;
  }

  const int nchunks = (s1 - s0 + 63) >> 6;
  const int iters = (nchunks + 3) >> 2;
  for (int it = 0; it < iters; ++it) {
    const int c = it * 4 + wave;
    const int cbase = s0 + c * 64;
    // scores: one key per lane
    const int j = cbase + lane;
    const bool valid = (c < nchunks) && (j < s1) && (j >= lo);
    float score[G];
    float nv = 0.0f;
    if (valid) {
      const int64_t page = (int64_t)btab[page_entry(a, j >> 4)] * a.num_kv_heads + h;
      const int o = j & 15;
      const uint8_t *kp = a.k_cache + page * KP;
      // record of coordinate chunk w: BITS code-plane words and the sign word
      // of 32 coordinates
      uint32_t wp[4][BITS + 1];
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int f = 0; f <= BITS; ++f) wp[w][f] = *reinterpret_cast<const uint32_t *>(kp + RB * (16 * w + o) + 4 * f);
      const float nk = (float)*reinterpret_cast<const _Float16 *>(kp + k_norm_off(BITS) + 2 * o);
      const float gm = (float)*reinterpret_cast<const _Float16 *>(kp + k_norm_off(BITS) + 32 + 2 * o);
      nv = (float)*reinterpret_cast<const _Float16 *>(a.v_cache + page * VP + v_norm_off(BITS) + 2 * o);
      float dk[G], ds[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        dk[g] = 0.0f;
        ds[g] = 0.0f;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll 8
        for (int bb = 0; bb < 32; ++bb) {
          const int i = w * 32 + bb;
          int idx = 0;
#pragma unroll
          for (int f = 0; f < BITS; ++f) idx |= ((wp[w][f] >> bb) & 1) << f;
          const float cv = lut[idx];
          const float sg = ((wp[w][BITS] >> bb) & 1) ? 1.0f : -1.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            dk[g] = fmaf(qp[g * 128 + i], cv, dk[g]);
            ds[g] = fmaf(sq[g * 128 + i], sg, ds[g]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) score[g] = cs * nk * fmaf(gm, ds[g], dk[g]);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) score[g] = -INFINITY;
    }
    // online softmax, wave-wide per head
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(m[g], wave_max(score[g]));
      const float p = (mn == -INFINITY) ? 0.0f : exp2f(score[g] - mn);
      const float corr = (mn == -INFINITY) ? 1.0f : exp2f(m[g] - mn);
      l[g] = l[g] * corr + wave_sum(p);
      acc0[g] *= corr;
      acc1[g] *= corr;
      m[g] = mn;
      pn[(wave * G + g) * 64 + lane] = p * nv;
    }
    lds_barrier();
    // values: lane owns coordinates lane and lane + 64
    if (c < nchunks) {
#pragma unroll 1
      for (int pg = 0; pg < 4; ++pg) {
        const int tok0 = cbase + pg * 16;
        if (tok0 >= s1) break;
        const uint8_t *vp = a.v_cache + ((int64_t)btab[page_entry(a, tok0 >> 4)] * a.num_kv_heads + h) * VP;
        // plane words of coordinates lane and lane + 64 (16 token bits each)
        uint32_t pa[BITS], pb[BITS];
#pragma unroll
        for (int f = 0; f < BITS; ++f) {
          pa[f] = *reinterpret_cast<const uint16_t *>(vp + kVPlane * f + 2 * lane);
          pb[f] = *reinterpret_cast<const uint16_t *>(vp + kVPlane * f + 128 + 2 * lane);
        }
#pragma unroll 4
        for (int tt = 0; tt < 16; ++tt) {
          int ia = 0, ib = 0;
#pragma unroll
          for (int f = 0; f < BITS; ++f) {
            ia |= ((pa[f] >> tt) & 1) << f;
            ib |= ((pb[f] >> tt) & 1) << f;
          }
          const float ca = lut[ia], cb = lut[ib];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pv = pn[(wave * G + g) * 64 + pg * 16 + tt];
            acc0[g] = fmaf(pv, ca, acc0[g]);
            acc1[g] = fmaf(pv, cb, acc1[g]);
          }
        }
      }
    }
    lds_barrier();
  }

  // combine the four waves, write this chunk's partial
  float *red = smem;  // [4][G][128], reuses the main-loop storage
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      red_m[wave][g] = m[g];
      red_l[wave][g] = l[g];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    red[(wave * G + g) * 128 + lane] = acc0[g];
    red[(wave * G + g) * 128 + lane + 64] = acc1[g];
  }
  lds_barrier();
  for (int idx = tid; idx < Gr * 128; idx += 256) {
    const int g = idx >> 7, d = idx & 127;
    float M = red_m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][g]);
    float Ls = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (red_m[w][g] == -INFINITY) ? 0.0f : exp2f(red_m[w][g] - M);
      Ls = fmaf(f, red_l[w][g], Ls);
      A = fmaf(f, red[(w * G + g) * 128 + d], A);
    }
    float *part = a.partials + ((row0 + g) * a.part_stride + split) * kPartStride;
    if (d == 0) {
      part[0] = M;
      part[1] = Ls;
    }
    part[4 + d] = A;
  }
}

// ---- 2'. split pass on the matrix cores (single-query decode, G <= 8) -----
// Both contractions run on the scaled f8f6f4 MFMA with the stored bits as the
// fp4 operand (b_split: one and_or per 8 values) and the float side split
// into four digits in four A rows: the query side in balanced base 32 as fp6
// codes (formed inside the pass, with scale * log2(e) folded in, so that
// scores come out in log2 units), the weights in base 16, also as fp6 codes
// (both contractions run at the fp6 x fp4 rate).
// With the bit-plane form of the levels, c[idx] = -(beta0 B0 + beta1 B1 +
// beta2 B2 + beta3 Bx) where Bx = B0 B1 B2 is the plane of b0^b1^b2:
//   <q', c[idx]> = sum_p <-beta_p q', B_p>        (4 MFMAs per page)
//   gamma <s, sigma> = gamma <-s, B_sign>          (1 MFMA per page)
//   o' = -sum_p beta_p sum_j w_j B_p,j  with w_j = p_j n_v,j  (4 planes)
//
// A workgroup serves one chunk of one KV head and all of its G query heads:
// T = ceil(G/4) head tiles of four heads, 4T waves.  The chunk is walked in
// tiles of 128 tokens (8 pages, K-blocks of two pages).  Wave w scores the
// page pair w%4 (K-block w%4) for head tile w/4, and in the value
// contraction owns 32/T coordinates for all T head tiles, so every wave runs
// 10 score and 8 value MFMAs per tile and builds each bit-plane operand once.
// Pages go HBM -> registers (two tiles ahead) -> LDS (three slots); each
// barrier interval holds the scores of tile i and the values of tile i-1.
//
// Weights: a scoring wave keeps a reference R per head (log2 units, moved
// only when a score exceeds it by 64), p = 2^(score - R), w = p n_v, and
// X = rint(w 2^(141-ex)) < 2^15 for ex the exponent field of the block's
// largest w.  The four base-16 digits of X are written to LDS as the bit
// patterns of f16 subnormals d 2^-24, which take no conversion on the
// scoring side; the value side turns 32 of them into one fp6 operand of the
// codes of d/8 with one conversion instruction (divisor 2^-21, which keeps
// subnormal inputs), and row r's E8M0 scale 2^(ex - 126 - 4r + R - Racc)
// restores its place value relative to the accumulator reference Racc.
// The value operand from b_split has the affine form alpha_v + beta_v b per
// register v; digits of K slots in registers 0..2 are negated (sign bit)
// and the offsets become one per-row correction, sum_k c_v A_k with
// c = (-5, -3, -1, 0) per register, taken by two MFMAs against constant
// operands (-4, -3, -1, 0) and (-1, 0, 0, 0): acc_p + corr = sum w (1 - 2b).

constexpr int kTilePages = 8;
constexpr int kMaxSplitTiles = 64;          // tiles of 128 tokens per workgroup (chunks up to 8192 tokens)
constexpr int kKRec = 1120;                 // per page: K planes and signs (1024) | K n (32) | K gamma (32) | V n (32)
constexpr int kVPair = 4 * 512 + 64;        // per page pair: [plane][coordinate] words (page a | page b << 16);
                                            // plane 3 takes the spare lanes' stores, +64 spreads the pairs over the banks
constexpr int kWqRow = 144;                 // 128 digits of one A row, padded (288-byte rows)
constexpr int kRefStep = 64;                // a reference moves when exceeded by 2^64

// Maximum over the 16 lanes of a row on integer keys that order like the
// floats (NaN-free inputs): no canonicalisation between the DPP steps.
__device__ __forceinline__ int float_key(float v) {
  const int b = __float_as_int(v);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ int row_max16_key(int k) {
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0xB1, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x4E, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(k, 0x141, 0xF, 0xF, false), 0x1B, 0xF, 0xF, false));
  return max(k, __builtin_amdgcn_mov_dpp(k, 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float v) {
  const int k = row_max16_key(float_key(v));
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += xchg1(v);
  v += xchg2(v);
  v += xchg4(v);
  return v + xchg8(v);
}
__device__ __forceinline__ float half_lo(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
// A value the compiler keeps in a vector register (wave-uniform constants of
// three-operand bit operations, which cannot take two scalar operands).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// b_split with its constants in vector registers: one v_and_or per register.
struct BSplitK {
  uint32_t m0, m1, m2, m3, c0, c1, c3;
};
__device__ __forceinline__ BSplitK bsplit_consts() {
  return BSplitK{in_vgpr(0x11111111u), in_vgpr(0x22222222u), in_vgpr(0x44444444u), in_vgpr(0x88888888u),
                 in_vgpr(0x66666666u), in_vgpr(0x44444444u), in_vgpr(0x22222222u)};
}
__device__ __forceinline__ v8i bsplit(uint32_t P, const BSplitK &k) {
  v8i b;
  b[0] = (int)((P & k.m0) | k.c0);
  b[1] = (int)((P & k.m1) | k.c1);
  b[2] = (int)(P & k.m2);
  b[3] = (int)((P & k.m3) | k.c3);
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// Maximum over the 16 lanes of a row for non-negative integer keys (0 is
// the identity, so the DPP moves fold into the max).
__device__ __forceinline__ int row_max16_nonneg(int k) {
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x141, 0xF, 0xF, true));  // row_half_mirror
  return max(k, __builtin_amdgcn_update_dpp(0, k, 0x140, 0xF, 0xF, true));  // row_mirror
}

// Loads of one tile by one wave into registers and their copies into LDS,
// addressed from a page base in scalar registers plus a fixed lane offset.
// Per page, the K part (used by the scores): code planes and signs (64
// lanes x 16 bytes), the K norms and residual norms (16 lanes x 4 bytes)
// and the V norms (8 lanes x 4 bytes); the V part (used by the value
// contraction): the V code planes (48 lanes x 16 bytes).  The K part of
// tile t is fetched three intervals ahead and copied to LDS one interval
// ahead; the V part is fetched two intervals ahead and copied in the
// interval of its own tile, so two LDS buffers of each suffice.  Role 2
// (T = 1) takes both parts of its page pair; with T = 2, role 0 (waves 0..3)
// takes the K planes and role 1 (waves 4..7) the rest of page pair w%4.  The
// role is a compile-time parameter, so that every loaded register has one
// producer and the counters of outstanding loads stay exact.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A wave-uniform byte pointer, kept in scalar registers so that loads take
// the scalar-base plus 32-bit lane-offset form.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}
typedef __attribute__((address_space(1))) const uint8_t gbyte;
template <typename V>
__device__ __forceinline__ V load_at(const uint8_t *base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(1))) V *>(
      reinterpret_cast<gbyte *>(reinterpret_cast<uint64_t>(base)) + off);
}
template <int R>
struct StageSet {
  u32x4 a[2];      // K planes (roles 0, 2) or V planes (role 1)
  u32x4 b[2];      // V planes (role 2)
  uint32_t t[4];   // K norm words, V norm words (roles 1, 2)
};
struct StagePtrs {
  const uint8_t *k_cache, *v_cache;
  int64_t hkv;
  int h, pr;
  uint32_t o16, o48, o16w, o8w;  // 16 lane; 16 (lane % 48); 4 (lane % 16); 4 (lane % 8)
};
template <int R>
__device__ __forceinline__ void load_k_part(StageSet<R> &S, const StagePtrs &P, int b0, int b1) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t blk = (e ? b1 : b0) * P.hkv + P.h;
    const uint8_t *kp = uniform_ptr(P.k_cache + blk * kKPage);
    if (R != 1) S.a[e] = load_at<u32x4>(kp, P.o16);
    if (R != 0) {
      S.t[e] = load_at<uint32_t>(kp + kKNorm, P.o16w);
      S.t[2 + e] = load_at<uint32_t>(uniform_ptr(P.v_cache + blk * kVPage + kVNorm), P.o8w);
    }
  }
}
template <int R>
__device__ __forceinline__ void load_v_part(StageSet<R> &S, const StagePtrs &P, int b0, int b1) {
  if (R == 0) return;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t blk = (e ? b1 : b0) * P.hkv + P.h;
    const u32x4 v = load_at<u32x4>(uniform_ptr(P.v_cache + blk * kVPage), P.o48);
    if (R == 2) S.b[e] = v;
    else S.a[e] = v;
  }
}
template <int R>
__device__ __forceinline__ void store_k_part(uint8_t *kbuf, const StageSet<R> &S, const StagePtrs &P, int lane) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint8_t *rec = kbuf + kKRec * (2 * P.pr + e);
    if (R != 1) *reinterpret_cast<u32x4 *>(rec + P.o16) = S.a[e];
    if (R != 0) {  // lanes 16.. and 8.. repeat the words of lanes l % 16, l % 8 (no lane branches)
      *reinterpret_cast<uint32_t *>(rec + 1024 + P.o16w) = S.t[e];
      *reinterpret_cast<uint32_t *>(rec + 1088 + P.o8w) = S.t[2 + e];
    }
  }
}
// V planes of the page pair, interleaved: word (plane, coordinate c) holds
// page a's 16 token bits in its low half and page b's in its high half.
template <int R>
__device__ __forceinline__ void store_v_part(uint8_t *vbuf, const StageSet<R> &S, const StagePtrs &P, int lane) {
  if (R == 0) return;
  const u32x4 va = R == 2 ? S.b[0] : S.a[0], vb = R == 2 ? S.b[1] : S.a[1];
  u32x4 lo, hi;
  lo[0] = __builtin_amdgcn_perm(vb[0], va[0], 0x05040100u);
  lo[1] = __builtin_amdgcn_perm(vb[0], va[0], 0x07060302u);
  lo[2] = __builtin_amdgcn_perm(vb[1], va[1], 0x05040100u);
  lo[3] = __builtin_amdgcn_perm(vb[1], va[1], 0x07060302u);
  hi[0] = __builtin_amdgcn_perm(vb[2], va[2], 0x05040100u);
  hi[1] = __builtin_amdgcn_perm(vb[2], va[2], 0x07060302u);
  hi[2] = __builtin_amdgcn_perm(vb[3], va[3], 0x05040100u);
  hi[3] = __builtin_amdgcn_perm(vb[3], va[3], 0x07060302u);
  // lane: plane lane/16, coordinates 8 (lane % 16) .. +7
  uint8_t *dst = vbuf + kVPair * P.pr + 512 * (lane >> 4) + 32 * (lane & 15);  // lanes 48..: spare plane
  *reinterpret_cast<u32x4 *>(dst) = lo;
  *reinterpret_cast<u32x4 *>(dst + 16) = hi;
}

// Scratch of the query operands (below), in the staging buffers and, where
// it is larger, the space after them.
template <int T>
struct QPrepLds {
  float qr[4 * T][kHeadDim];           // q' = H q (zero rows for absent heads)
  float sv[4 * T][kQjlDim];            // s = alpha S q
  _Float16 qh[4 * T][kHeadDim];        // q' as f16 hi + lo halves in slot order
  _Float16 ql[4 * T][kHeadDim];        //   (slot s <-> coordinate 16 (s % 8) + s / 8)
  _Float16 codes[4 * T][5][4][128];    // [head][plane][digit][K slot] digit values d f (exact)
  int pe[4 * T][5];                    // per head and plane: E, or INT_MIN for a zero plane
};
constexpr int kStageBytes = 2 * kTilePages * kKRec + 2 * 4 * kVPair;
template <int T>
constexpr int qprep_pad() {
  return (int)sizeof(QPrepLds<T>) > kStageBytes ? (int)sizeof(QPrepLds<T>) - kStageBytes : 16;
}

template <int T>
struct SplitLds {
  int ids[kMaxSplitTiles][kTilePages];      // block ids of the chunk's pages
  uint8_t kbuf[2][kTilePages * kKRec];
  uint8_t vbuf[2][4 * kVPair];
  uint8_t qpad[qprep_pad<T>()];             // rest of the query scratch
  alignas(16) uint16_t wq[2][T][16][kWqRow];  // [buffer][head tile][head * 4 + digit][K slot] digit bits as f16 subnormals
  int2 stats[2][T][4][4];        // [buffer][head tile][head][K-block]: (exponent field, R bits)
  float lred[T][4][4][2];        // [head tile][head][K-block]: (probability sum, R)
  float cred[4 * T][T][4][4];    // [wave][head tile][head][digit]: correction partials
};

static_assert(offsetof(SplitLds<1>, wq) - offsetof(SplitLds<1>, kbuf) >= sizeof(QPrepLds<1>), "query scratch");
static_assert(offsetof(SplitLds<2>, wq) - offsetof(SplitLds<2>, kbuf) >= sizeof(QPrepLds<2>), "query scratch");

template <bool B>
using flag = std::integral_constant<bool, B>;

// ---- query operands inside the split pass ------------------------------------
// The matrix-core split pass forms the query-side operands of its G heads
// itself while its first tiles are in flight: q' = H q, s = alpha S q, and
// the A operands of the score contraction: rows (head, digit r), for x the
// plane's values times scale * log2(e) (scores in log2 units).  With 2^E
// bounding |x| over the head, Y = rint(x 2^(19-E)) is written in balanced
// base 32, Y = d0 2^15 + d1 2^10 + d2 2^5 + d3 with every |d_r| <= 16, stored
// as the fp6 e2m3 code of d_r/8 (exact), and row r carries it with scale
// 2^(E-4-5r+3): x to 2^-20 of the head's largest magnitude.  Logits of keys
// with large norms need these 19 bits; 16 (base-16 digits) leave errors near
// 1e-3 in peaked rows.  Every workgroup of a (sequence, KV head) repeats this
// small amount of work (16 K multiply-adds per head) instead of waiting for a
// separate launch and a round trip of its results through memory.  The
// scratch space aliases the staging buffers, which are first written after it.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v32h __attribute__((ext_vector_type(32)));
typedef int v16i __attribute__((ext_vector_type(16)));

// 32 f16 values at p (16-byte aligned) as one fp6 e2m3 operand, value / div
// (code s at bits 6s .. 6s+5; the conversion keeps f16 subnormal inputs).
__device__ __forceinline__ v8i fp6_operand(const uint16_t *p, float div) {
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
  const uint4 a = q[0], b = q[1], c = q[2], d = q[3];
  const v16i w = v16i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w,
                      (int)c.x, (int)c.y, (int)c.z, (int)c.w, (int)d.x, (int)d.y, (int)d.z, (int)d.w};
  const auto r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(__builtin_bit_cast(v32h, w), div);
  return v8i{(int)r[0], (int)r[1], (int)r[2], (int)r[3], (int)r[4], (int)r[5], 0, 0};
}

// Query rows of a (sequence, KV head) workgroup of the matrix-core pass:
// row = i G + g for position t = pos0 + i of the q_len new ones and head g
// of the group.  Its output row is (b q_len + t) Hq + h G + g, and it sees
// the keys before L - q_len + t + 1 (multi-token verify is causal over the
// new ones).
// (The host bounds the group index below 2^31: 32-bit division.)
__device__ __forceinline__ int64_t query_out_row(const DecodeArgs &a, int64_t grp, int row) {
  const int G = a.group;
  const int g32 = (int)grp, b = g32 / a.num_kv_heads, h = g32 - b * a.num_kv_heads;
  return ((int64_t)b * a.q_len + a.pos0 + row / G) * a.num_q_heads + h * G + row % G;
}


// Loads issued first in the workgroup, so that waiting for them does not wait
// for the tile loads issued after them: wave w's q elements lane and lane + 64
// of head w (one unconditional dword each, converted later; an absent head
// repeats the last one) and, for a wave that forms part of s (waves 0..3),
// its rows 32 w .. 32 w + 31 of S H as the f16 operands of the projection.
template <bool PROJ>
struct QPrepRegs {
  uint32_t qw[2];
  uint4 sh[PROJ ? 16 : 1];
};
// The projection operands alone (they depend on no argument of the call's
// plan, so they can be requested before it is known).
template <bool PROJ>
__device__ __forceinline__ void qprep_load_sh(const DecodeArgs &a, int wave, int lane, QPrepRegs<PROJ> &R) {
  if constexpr (PROJ) {
    const uint4 *shop = reinterpret_cast<const uint4 *>(a.SHop) + wave * 2 * 4 * 2 * 64 + lane;
#pragma unroll
    for (int e = 0; e < 16; ++e) R.sh[e] = shop[e * 64];
  }
}
// The query words alone (hbase: the first query row of the wave's head tile).
template <bool PROJ>
__device__ __forceinline__ void qprep_load_q(const DecodeArgs &a, int64_t grp, int wave, int lane, QPrepRegs<PROJ> &R,
                                             int hbase = 0) {
  const int rows = a.group * a.pos_count;
  const bool f32 = a.q_dtype == TQ_F32;
  const int64_t row = query_out_row(a, grp, min(hbase + wave, rows - 1));
  const uint32_t *base = static_cast<const uint32_t *>(a.q);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t idx = row * kHeadDim + lane + 64 * j;
    R.qw[j] = base[f32 ? idx : (idx >> 1)];
  }
}
template <bool PROJ>
__device__ __forceinline__ void qprep_loads(const DecodeArgs &a, int64_t grp, int wave, int lane, QPrepRegs<PROJ> &R) {
  const int rows = a.group * a.pos_count;
  const bool f32 = a.q_dtype == TQ_F32;
  const int64_t row = query_out_row(a, grp, min(wave, rows - 1));
  const uint32_t *base = static_cast<const uint32_t *>(a.q);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t idx = row * kHeadDim + lane + 64 * j;
    R.qw[j] = base[f32 ? idx : (idx >> 1)];
  }
  if constexpr (PROJ) {
    const uint4 *shop = reinterpret_cast<const uint4 *>(a.SHop) + wave * 2 * 4 * 2 * 64 + lane;
#pragma unroll
    for (int e = 0; e < 16; ++e) R.sh[e] = shop[e * 64];
  }
}

// The operands, for the head tiles NU the calling wave scores (every wave of
// the workgroup runs this; with TAIL it ends on a barrier after which the
// scratch space may be reused).  Wave w rotates and digitises head w of the
// workgroup's heads, which start at query row hbase of the group (a head tile
// of its own when a separate launch forms one tile's operands).  The
// operands and start values of code planes 0..3 are formed as soon as their
// digits are (beside the projection); the sign plane's once s is.
template <int T, int NU, bool PACK, bool PROJ, bool TAIL = true>
__device__ __forceinline__ void qprep_compute(const DecodeArgs &a, QPrepLds<T> &L, const QPrepRegs<PROJ> &R, int tid,
                                              int wave, const int (&tiles)[NU], v8i (&Aq)[NU][5],
                                              int (&scq)[NU][5], v4f (&cinit)[NU], v4f (&qinit)[NU],
                                              int hbase = 0) {
  const int lane = tid & 63, rows = a.group * a.pos_count - hbase;
  float x[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t w = R.qw[j];
    float v;
    if (a.q_dtype == TQ_F32) {
      v = __uint_as_float(w);
    } else {
      const uint32_t hb = (lane & 1) ? (w >> 16) : (w & 0xFFFFu);  // element lane + 64 j has the parity of lane
      v = a.q_dtype == TQ_F16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)hb) : __uint_as_float(hb << 16);
    }
    x[j] = wave < rows ? v : 0.0f;
  }
  wave_fwht128(x[0], x[1], lane);
  L.qr[wave][lane] = x[0];
  L.qr[wave][lane + 64] = x[1];
  const float hq = wave_max(fmaxf(fabsf(x[0]), fabsf(x[1])));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = lane + 64 * j, sl = 8 * (c & 15) + (c >> 4);
    const _Float16 hi = (_Float16)x[j];
    L.qh[wave][sl] = hi;
    L.ql[wave][sl] = (_Float16)(x[j] - (float)hi);
  }
  // wave w: the digits of head w.  Planes 0..3 need only the wave's own q'
  // (LDS operations of a wave complete in order), so they are formed before
  // the first barrier; plane 4 waits for the projection.
  float beta[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) beta[p] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.beta[p])));
  const float cs = a.scale * kLog2e;
  // Y = rint(x 2^(19-E)) = d0 2^15 + d1 2^10 + d2 2^5 + d3, |d_r| <= 16
  auto digits = [&](int p, int kap, float x, int pe) __attribute__((always_inline)) {
    const bool pz = pe != INT_MIN;
    const float f = b_split_factor(kap);
    const float y = pz ? rintf(ldexpf(x, 19 - (pz ? pe : 0))) : 0.0f;
    const float d0 = rintf(y * 0x1p-15f);
    float rem = y - d0 * 32768.0f;
    const float d1 = rintf(rem * 0x1p-10f);
    rem -= d1 * 1024.0f;
    const float d2 = rintf(rem * 0.03125f);
    const float d3 = rem - d2 * 32.0f;
    L.codes[wave][p][0][kap] = (_Float16)(d0 * f);
    L.codes[wave][p][1][kap] = (_Float16)(d1 * f);
    L.codes[wave][p][2][kap] = (_Float16)(d2 * f);
    L.codes[wave][p][3][kap] = (_Float16)(d3 * f);
  };
  {
    int pe[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float M = cs * fabsf(beta[p]) * hq;
      pe[p] = M > 0.0f ? max(bound_exponent(M), -100) : INT_MIN;
    }
    if (lane < 4) L.pe[wave][lane] = lane == 0 ? pe[0] : lane == 1 ? pe[1] : lane == 2 ? pe[2] : pe[3];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const int kap = lane + 64 * hk;
      const float qv = L.qr[wave][b_coord(kap)];
#pragma unroll
      for (int p = 0; p < 4; ++p) digits(p, kap, -cs * beta[p] * qv, pe[p]);
    }
  }
  lds_barrier();
  // this lane's operand rows: (head 4u + gp, digit r), K-block ga.  The
  // start values (see b_split), sum_k (1 - f_v alpha_v) A_k = -sum_k w_v A_k
  // with w_v = 5, 3, 1, 0, are two matrix ops per plane against the constant
  // operands -(4, 3, 1, 0) and -(1, 0, 0, 0) (e2m1 codes E, D, A and A).
  const int ga = lane >> 4, gp = (lane & 15) >> 2, r = lane & 3;
  const v8i W1 = v8i{(int)0xEEEEEEEEu, (int)0xDDDDDDDDu, (int)0xAAAAAAAAu, 0, 0, 0, 0, 0};
  const v8i W2 = v8i{(int)0xAAAAAAAAu, 0, 0, 0, 0, 0, 0, 0};
  auto pack_plane = [&](int n, int p) __attribute__((always_inline)) {
    const int hd = 4 * tiles[n] + gp;
    // the 32 digit values of K slots 32 ga .. +31, as codes of d / 8
    Aq[n][p] = fp6_operand(reinterpret_cast<const uint16_t *>(&L.codes[hd][p][r][32 * ga]), 8.0f);
    const int E = L.pe[hd][p];
    scq[n][p] = E != INT_MIN ? min(E - 4 - 5 * r + kFp6Exp + kE8M0One, 254) : kE8M0One;
  };
#pragma unroll
  for (int n = 0; n < (PACK ? NU : 0); ++n) {
#pragma unroll
    for (int p = 0; p < 4; ++p) pack_plane(n, p);
    v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      c = mfma_f6f4(Aq[n][p], W1, c, scq[n][p]);
      c = mfma_f6f4(Aq[n][p], W2, c, scq[n][p]);
    }
    cinit[n] = c;
  }
  if constexpr (PROJ) {
    // s = alpha (S H) q' for rows 32 w .. 32 w + 31, all heads: three f16
    // passes (hi hi + hi lo + lo hi, ~22 bits); A rows past the heads are zero
    const int hr = lane & 15;
    const bool live = hr < 4 * T;
    v4f z[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = live ? hr : 0, col = 32 * k + 8 * (lane >> 4);
      const uint4 h4 = *reinterpret_cast<const uint4 *>(&L.qh[row][col]);
      const uint4 l4 = *reinterpret_cast<const uint4 *>(&L.ql[row][col]);
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
      const v8h ah = __builtin_bit_cast(v8h, live ? h4 : zero), al = __builtin_bit_cast(v8h, live ? l4 : zero);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v8h bh = __builtin_bit_cast(v8h, R.sh[(u * 4 + k) * 2]), bl = __builtin_bit_cast(v8h, R.sh[(u * 4 + k) * 2 + 1]);
        z[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, z[u], 0, 0, 0);
        z[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, z[u], 0, 0, 0);
        z[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, z[u], 0, 0, 0);
      }
    }
    // lane l, register i: head 4 (l / 16) + i, row 16 (2 w + u) + l % 16
    const float qjl = a.cb.qjl_scale;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = 4 * (lane >> 4) + i;
        if (hd < 4 * T) L.sv[hd][16 * (2 * wave + u) + (lane & 15)] = qjl * z[u][i];
      }
  }
  lds_barrier();
  {
    const float hs = wave_max(fmaxf(fabsf(L.sv[wave][lane]), fabsf(L.sv[wave][lane + 64])));
    const float M = cs * hs;
    const int pe4 = M > 0.0f ? max(bound_exponent(M), -100) : INT_MIN;
    if (lane == 4) L.pe[wave][4] = pe4;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const int kap = lane + 64 * hk;
      digits(4, kap, -cs * L.sv[wave][b_coord(kap)], pe4);
    }
  }
  lds_barrier();
#pragma unroll
  for (int n = 0; n < (PACK ? NU : 0); ++n) {
    pack_plane(n, 4);
    const v4f z = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    qinit[n] = mfma_f6f4(Aq[n][4], W2, mfma_f6f4(Aq[n][4], W1, z, scq[n][4]), scq[n][4]);
  }
  if constexpr (TAIL) lds_barrier();  // the scratch space is free again
}


// Five to eight heads per KV head (two head tiles): the waves specialise.
// Waves 0..3 (role 0) score page pair w of every tile for both head tiles,
// so each K page is expanded into operands once, and stage the K planes;
// waves 4..7 (role 1) contract the values of coordinates 32(w-4) .. +31 for
// both head tiles and stage the norms and V planes.  The two waves that share
// a SIMD then issue different mixes (vector-heavy scores, matrix-heavy
// values) and overlap, where identical waves run the same phases in lock
// step.  Intervals, buffers and records are the ones described above.
template <int R>
__device__ __attribute__((always_inline)) void split_body_ws(const DecodeArgs &a, SplitLds<2> &sm, int b, int h,
                                                             int split, int s0, int s1) {
  constexpr int T = 2;
  constexpr int NW = 8;  // waves
  constexpr int NJ = 2;  // value N-tiles (16 coordinates) per value wave
  const int L = clamped_context(a, b);
  // query rows (positions x heads); every row sees the keys before s1v, row
  // r those before min(s1, L - q_len + pos0 + r / G + 1)
  const int qlen = a.q_len - a.pos0, nrows = a.group * a.pos_count;
  const int s1v = min(s1, L - qlen + 1);
  // with a window, every row sees the keys from s0v on (the latest row's lower end)
  const int s0v = window_low(a, L - qlen + (a.group * a.pos_count - 1) / a.group + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sq = wave & 3;  // role 0: page pair (K-block); role 1: coordinate block
  const int t16 = lane & 15, grow = lane >> 4;
  const int64_t grp = (int64_t)b * a.num_kv_heads + h;
  const int G = a.group;
  const int ntiles = min((s1 - s0 + 127) >> 7, kMaxSplitTiles);  // the host caps chunks at 64 tiles

  {
    const int32_t *btab = a.block_tables + (int64_t)b * a.max_blocks;
    for (int idx = tid; idx < ntiles * kTilePages; idx += 64 * NW) {
      const int tile0 = s0 + 128 * (idx >> 3);
      const int tok = tile0 + 16 * (idx & 7);
      sm.ids[idx >> 3][idx & 7] = btab[page_entry(a, (tok < s1 ? tok : tile0) >> 4)];
    }
  }

  // role 0: query-side operands of the score contraction, both head tiles,
  // formed in the prologue; their loads go out first
  QPrepRegs<R == 0> qpr;
  qprep_loads<R == 0>(a, grp, wave, lane, qpr);
  v8i Aq[T][5];
  int scq[T][5];
  v4f cinit[T], qinit[T];
  float beta[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) beta[p] = uniform(a.cb.beta[p]);
  const BSplitK bk = bsplit_consts();
  const uint32_t nib = in_vgpr(0x000F000Fu);
  const uint32_t s80 = in_vgpr((t16 & 3) == 3 ? 0u : 0x80008000u);
  const int kap0 = 8 * (t16 & 3) + (t16 >> 2);
  const StagePtrs sp{a.k_cache, a.v_cache, (int64_t)a.num_kv_heads, h, sq, 16u * (uint32_t)lane,
                     16u * (uint32_t)(lane % 48), 4u * (uint32_t)t16, 4u * (uint32_t)(lane & 7)};
  auto pair_ids = [&](int k, int &b0, int &b1) __attribute__((always_inline)) {
    const int2 v = *reinterpret_cast<const int2 *>(&sm.ids[k][2 * sq]);
    b0 = __builtin_amdgcn_readfirstlane(v.x);
    b1 = __builtin_amdgcn_readfirstlane(v.y);
  };

  // role 0 state (lane: head grow of tile u, token t16)
  float rl[T], lsum[T];
  // role 1 state (lane: A row (head gA, digit rA), K-block kb; C rows head grow)
  const int gA = t16 >> 2, rA = lane & 3, kb = grow;
  float raA[T], raC[T];
  v4f acc[T][4][NJ];
  v4f corr[T];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    rl[u] = -INFINITY;
    lsum[u] = 0.0f;
    corr[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    raA[u] = raC[u] = -INFINITY;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[u][p][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // role 1: E8M0 scales of the weight rows in buffer bf
  auto value_scales = [&](int bf, int (&sw)[T]) __attribute__((always_inline)) {
    int2 st[T];
    bool move = false;
#pragma unroll
    for (int u = 0; u < T; ++u) {
      st[u] = sm.stats[bf][u][gA][kb];
      move |= __int_as_float(st[u].y) > raA[u] + (float)kRefStep;
    }
    if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
      for (int u = 0; u < T; ++u) {
        float MA = -INFINITY, MC = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          MA = fmaxf(MA, __int_as_float(sm.stats[bf][u][gA][q].y));
          MC = fmaxf(MC, __int_as_float(sm.stats[bf][u][grow][q].y));
        }
        if (MA > raA[u] + (float)kRefStep) raA[u] = MA;
        float fc = 1.0f;
        if (MC > raC[u] + (float)kRefStep) {
          fc = raC[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(raC[u] - MC);
          raC[u] = MC;
        }
        corr[u] *= fc;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[u][p][j] *= fc;
      }
    }
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const float d = fmaxf(__int_as_float(st[u].y) - raA[u], -300.0f);  // NaN (both -inf) -> -300
      sw[u] = min(max(st[u].x + 1 - 4 * rA + (int)d, 0), 254);
    }
  };

  // One barrier interval: the staging of both roles, then
  // role 0 scores tile k, role 1 contracts the values of tile k-1 (without
  // scores: of tile k).
  auto interval = [&](auto HS, auto HV, auto PAR, StageSet<R> &SK, StageSet<R> &SV, int k)
                      __attribute__((always_inline)) {
    constexpr bool has_s = decltype(HS)::value, has_v = decltype(HV)::value;
    constexpr int par = decltype(PAR)::value;
    constexpr int bs = par, bv = has_s ? (par ^ 1) : par;
    const int kv = has_s ? k - 1 : k;
    if constexpr (has_s) {
      int k3a, k3b, k2a, k2b;
      pair_ids(min(k + 3, ntiles - 1), k3a, k3b);
      pair_ids(min(k + 2, ntiles - 1), k2a, k2b);
      store_v_part<R>(sm.vbuf[par], SV, sp, lane);
      store_k_part<R>(sm.kbuf[par ^ 1], SK, sp, lane);
      load_k_part<R>(SK, sp, k3a, k3b);
      load_v_part<R>(SV, sp, k2a, k2b);
    }
    if constexpr (R == 0 && has_s) {
      uint32_t kw[2][4];
      uint32_t nrm[2][3];  // half bits: n_k, gamma, n_v
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint8_t *rec = sm.kbuf[bs] + kKRec * (2 * sq + e);
        const u32x4 kr = *reinterpret_cast<const u32x4 *>(rec + k_record(grow, t16));  // planes 0..2, signs
        kw[e][0] = kr[0];
        kw[e][1] = kr[1];
        kw[e][2] = kr[2];
        kw[e][3] = kr[3];
        const uint16_t *nr = reinterpret_cast<const uint16_t *>(rec + 1024);
        nrm[e][0] = nr[t16];
        nrm[e][1] = nr[16 + t16];
        nrm[e][2] = nr[32 + t16];
      }
      // each page's operands once, for both head tiles
      v4f cc[T][2], qq[T][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w0 = kw[e][0], w1 = kw[e][1], w2 = kw[e][2], w3 = kw[e][3];
        const v8i B0 = bsplit(w0, bk), B1 = bsplit(w1, bk), B2 = bsplit(w2, bk);
        const v8i Bx = bsplit(w0 ^ w1 ^ w2, bk), Bs = bsplit(w3, bk);
#pragma unroll
        for (int u = 0; u < T; ++u) {
          v4f c = mfma_f6f4(Aq[u][0], B0, cinit[u], scq[u][0]);
          c = mfma_f6f4(Aq[u][1], B1, c, scq[u][1]);
          c = mfma_f6f4(Aq[u][2], B2, c, scq[u][2]);
          cc[u][e] = mfma_f6f4(Aq[u][3], Bx, c, scq[u][3]);
          qq[u][e] = mfma_f6f4(Aq[u][4], Bs, qinit[u], scq[u][4]);
          pin_result(cc[u][e]);
          pin_result(qq[u][e]);
        }
      }
      // uniform: a tile some row does not see whole
      const bool partial = s0 + 128 * (k + 1) > s1v || s0 + 128 * k < s0v;
#pragma unroll
      for (int u = 0; u < T; ++u) {
        float inner[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const v4f &c = cc[u][e], &q = qq[u][e];
          const float code = (c[0] + c[1]) + (c[2] + c[3]);
          const float qj = (q[0] + q[1]) + (q[2] + q[3]);
          inner[e] = fmaf(half_lo(nrm[e][1]), qj, code);
        }
        const float lsum0 = lsum[u];
        auto weights = [&](float x0, float x1, bool v0, bool v1) __attribute__((always_inline)) {
          const float p0 = __builtin_amdgcn_exp2f(x0), p1 = __builtin_amdgcn_exp2f(x1);
          lsum[u] += p0 + p1;
          const float w0 = v0 ? p0 * half_lo(nrm[0][2]) : 0.0f;
          const float w1 = v1 ? p1 * half_lo(nrm[1][2]) : 0.0f;
          const int mk = row_max16_nonneg(max(__float_as_int(w0), __float_as_int(w1)));  // w >= 0
          const uint32_t exb = max((uint32_t)mk & 0x7F800000u, 14u << 23);
          const float mult = __uint_as_float(0x86000000u - exb);  // 2^(141 - ex)
          const uint32_t X0 = __float_as_uint(fmaf(w0, mult, 8388608.0f));
          const uint32_t X1 = __float_as_uint(fmaf(w1, mult, 8388608.0f));
          const uint32_t XX = __builtin_amdgcn_perm(X1, X0, 0x05040100u);  // X0 lo16 | X1 lo16 << 16
          uint16_t *wr = &sm.wq[bs][u][4 * grow][32 * sq + kap0];
#pragma unroll
          for (int r = 0; r < 4; ++r) {  // digit r (place 16^(3-r)) of both tokens, with the slot's sign
            const uint32_t D = ((XX >> (12 - 4 * r)) & nib) | s80;
            wr[r * kWqRow] = (uint16_t)D;
            wr[r * kWqRow + 4] = (uint16_t)(D >> 16);
          }
          sm.stats[bs][u][grow][sq] = make_int2((int)(exb >> 23), __float_as_int(rl[u]));
        };
        const float x0 = fmaf(half_lo(nrm[0][0]), inner[0], -rl[u]);
        const float x1 = fmaf(half_lo(nrm[1][0]), inner[1], -rl[u]);
        weights(x0, x1, true, true);
        if (__builtin_amdgcn_ballot_w64(x0 > (float)kRefStep || x1 > (float)kRefStep) || partial) {
          const int tok0 = s0 + 128 * k + 32 * sq + t16;
          const int hi = L - qlen + (4 * u + grow) / G + 1;  // the lane's row
          const int lim = min(s1, hi), lo = window_low(a, hi);
          const bool v0 = tok0 < lim && tok0 >= lo, v1 = tok0 + 16 < lim && tok0 + 16 >= lo;
          const float r0 = v0 ? half_lo(nrm[0][0]) * inner[0] : -INFINITY;
          const float r1 = v1 ? half_lo(nrm[1][0]) * inner[1] : -INFINITY;
          const float mh = row_max16(fmaxf(r0, r1));
          const float nr = fmaxf(rl[u], ceilf(mh));
          lsum[u] = lsum0;
          if (nr > rl[u] && nr - rl[u] > 0.0f) {
            lsum[u] = rl[u] == -INFINITY ? 0.0f : lsum[u] * __builtin_amdgcn_exp2f(rl[u] - nr);
            rl[u] = nr;
          }
          weights(r0 == -INFINITY ? -INFINITY : r0 - rl[u], r1 == -INFINITY ? -INFINITY : r1 - rl[u], v0, v1);
        }
      }
    }
    if constexpr (R == 1 && has_v) {
      int sw[T];
      value_scales(bv, sw);
      v8i Aw[T];
#pragma unroll
      for (int u = 0; u < T; ++u) Aw[u] = fp6_operand(&sm.wq[bv][u][4 * gA + rA][32 * kb], 0x1p-21f);  // d 2^-24 -> d/8
      const uint32_t *vw = reinterpret_cast<const uint32_t *>(sm.vbuf[bv] + kVPair * kb);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = 16 * (NJ * sq + j) + t16;
        const uint32_t W0 = vw[c], W1 = vw[128 + c], W2 = vw[256 + c];
        const v8i V0 = bsplit(W0, bk), V1 = bsplit(W1, bk), V2 = bsplit(W2, bk), Vx = bsplit(W0 ^ W1 ^ W2, bk);
#pragma unroll
        for (int u = 0; u < T; ++u) {
          acc[u][0][j] = mfma_f6f4(Aw[u], V0, acc[u][0][j], sw[u]);
          acc[u][1][j] = mfma_f6f4(Aw[u], V1, acc[u][1][j], sw[u]);
          acc[u][2][j] = mfma_f6f4(Aw[u], V2, acc[u][2][j], sw[u]);
          acc[u][3][j] = mfma_f6f4(Aw[u], Vx, acc[u][3][j], sw[u]);
        }
      }
      if (kv % 4 == sq) {  // uniform: the offsets of b_split, one value wave per tile
        const v8i C1 = v8i{(int)0xEEEEEEEEu, (int)0xDDDDDDDDu, (int)0xAAAAAAAAu, 0, 0, 0, 0, 0};
        const v8i C2 = v8i{(int)0xAAAAAAAAu, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < T; ++u) {
          corr[u] = mfma_f6f4(Aw[u], C1, corr[u], sw[u]);
          corr[u] = mfma_f6f4(Aw[u], C2, corr[u], sw[u]);
        }
      }
    }
  };

  for (int i = tid; i < T * 16 * kWqRow / 2; i += 64 * NW) reinterpret_cast<uint32_t *>(&sm.wq[1][0][0][0])[i] = 0u;
  if (tid < T * 16) (&sm.stats[1][0][0][0])[tid] = make_int2(0, __float_as_int(-INFINITY));
  lds_barrier();  // block ids, buffer 1
  StageSet<R> SA, SB;
  {
    int b0, b1, c0, c1, d0, d1;
    pair_ids(0, b0, b1);
    pair_ids(min(1, ntiles - 1), c0, c1);
    pair_ids(min(2, ntiles - 1), d0, d1);
    load_k_part<R>(SA, sp, b0, b1);
    __builtin_amdgcn_sched_barrier(0);
    load_k_part<R>(SB, sp, c0, c1);
    load_v_part<R>(SA, sp, b0, b1);
    __builtin_amdgcn_sched_barrier(0);
    // the query operands while these tiles are in flight (scratch in the
    // staging buffers, which are written from here on); role 1 takes part in
    // the work and the barriers but keeps no operands
    {
      const int tiles[2] = {0, 1};
      qprep_compute<T, 2, R == 0, R == 0>(a, *reinterpret_cast<QPrepLds<T> *>(&sm.kbuf[0][0]), qpr, tid, wave, tiles, Aq,
                                  scq, cinit, qinit);
    }
    store_k_part<R>(sm.kbuf[0], SA, sp, lane);
    load_k_part<R>(SA, sp, d0, d1);
    load_v_part<R>(SB, sp, c0, c1);
    __builtin_amdgcn_sched_barrier(0);
  }
  lds_barrier();
  int k = 0;
  for (; k + 1 < ntiles; k += 2) {
    interval(flag<true>{}, flag<true>{}, std::integral_constant<int, 0>{}, SB, SA, k);
    lds_barrier();
    interval(flag<true>{}, flag<true>{}, std::integral_constant<int, 1>{}, SA, SB, k + 1);
    lds_barrier();
  }
  if (k < ntiles) {  // uniform
    interval(flag<true>{}, flag<true>{}, std::integral_constant<int, 0>{}, SB, SA, k);
    lds_barrier();
  }
  if ((ntiles - 1) & 1)
    interval(flag<false>{}, flag<true>{}, std::integral_constant<int, 1>{}, SA, SB, ntiles - 1);
  else
    interval(flag<false>{}, flag<true>{}, std::integral_constant<int, 0>{}, SA, SB, ntiles - 1);
#pragma unroll
  for (int u = 0; u < T; ++u) {
    asm volatile("" : "+v"(corr[u]));
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[u][p][j]));
  }

  if constexpr (R == 0) {  // probability sums per head
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const float ls = row_sum16(lsum[u]);
      if (t16 == 0) {
        sm.lred[u][grow][sq][0] = ls;
        sm.lred[u][grow][sq][1] = rl[u];
      }
    }
  } else {  // correction partials per value wave
#pragma unroll
    for (int u = 0; u < T; ++u)
      if (t16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.cred[sq][u][grow][i] = corr[u][i];
      }
  }
  lds_barrier();
  if constexpr (R == 1) {
    const float bsum = (beta[0] + beta[1]) + (beta[2] + beta[3]);
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const int g = 4 * u + grow;  // C rows of this lane: row grow of tile u
      if (g >= nrows) continue;
      const float ra = raC[u];
      float cs = 0.0f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv)
#pragma unroll
        for (int i = 0; i < 4; ++i) cs += sm.cred[wv][u][grow][i];
      float *part = a.partials + (query_out_row(a, grp, g) * a.part_stride + split) * kPartStride;
      if (sq == 0 && t16 == 0) {
        float l = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float rq = sm.lred[u][grow][q][1];
          if (rq != -INFINITY) l += sm.lred[u][grow][q][0] * __builtin_amdgcn_exp2f(rq - ra);
        }
        part[0] = ra;
        part[1] = l;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float o = -bsum * cs;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const v4f &c = acc[u][p][j];
          o = fmaf(-beta[p], (c[0] + c[1]) + (c[2] + c[3]), o);
        }
        part[4 + 16 * (NJ * sq + j) + t16] = o;
      }
    }
  }
}

// One workgroup per range of the balanced plan.
template <int T>
__global__ __launch_bounds__(256 * T, T == 1 ? 2 : 1) void split_mfma_kernel(DecodeArgs a0) {
  __shared__ __align__(16) SplitLds<T> sm;
  // a verify block's position groups (pos_count positions each) share one
  // launch: workgroup i takes group i % groups and range i / groups, so the
  // groups of one range run side by side and read its pages together
  const int groups = (a0.q_len - a0.pos0 + a0.pos_count - 1) / a0.pos_count;
  const int pg = (int)blockIdx.x % groups, wid = (int)blockIdx.x / groups;
  DecodeArgs a = a0;
  a.pos0 = a0.pos0 + pg * a0.pos_count;
  a.pos_count = min(a0.pos_count, a0.q_len - a.pos0);
  const int t0 = seq_tiles(a, threadIdx.x & 63);
  const int per = bal_per(a, t0);
  int b, h, j, Tb;
  bal_locate(a, t0, per, wid, b, h, j, Tb);
  if (b >= a.num_seqs) return;  // uniform: past the last range
  const int L = clamped_context(a, b), base = seq_base(a, L);
  const int s0 = base + 128 * per * j, s1 = min(base + 128 * per * (j + 1), L);
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)  // uniform: the wave's role
    split_body_ws<0>(a, sm, b, h, j, s0, s1);
  else
    split_body_ws<1>(a, sm, b, h, j, s0, s1);
}

// ---- 2''. exact hot window ---------------------------------------------------
// The recent tokens a deployment keeps uncompressed (the SwiftLM README
// compresses only past 2,048 tokens, its --turbo-kv option row) enter the
// same softmax as the compressed history (its note on --turbo-kv recall):
// this pass turns window chunks of kHotChunk tokens into partial records of
// the same form as the split passes (m in log2 units, l, acc' in the rotated
// domain), placed right after each row's compressed records, and the merge
// combines them all.  Single-query decode: every window token is visible.
//
// A workgroup takes one (sequence, KV head, 64-token chunk) and the G <= 16
// query heads of the group; wave w takes tokens 16w .. 16w + 15 of the chunk:
//   * scores S = Q K^T on the matrix cores (16x16x32, bf16 or f16 as the
//     window is stored; Q = scale log2(e) q as hi + lo halves of that type,
//     rows past G zero): lane l reads 16 bytes of token l % 16's row per K
//     step straight into the B operand, so a wave's 16 rows are read whole;
//     f32 windows run as three bf16 pieces of K against Q hi + lo;
//   * the heads' maxima and sums over the chunk meet in LDS; p goes to LDS;
//   * p v on the vector ALU: lane l owns coordinates 2l, 2l + 1 and reads
//     each of its 16 tokens' rows as one coalesced 256-byte (bf16/f16) or
//     512-byte (f32) wave load;
//   * the waves' sums meet in LDS and each head's is rotated once (H is its
//     own inverse, so the merge's inverse rotation returns it).
template <int DT>
__device__ __forceinline__ float hot_elem(uint32_t hb) {
  return DT == TQ_F16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)hb) : __uint_as_float(hb << 16);
}
typedef short v8sh __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int DT>
__device__ __forceinline__ v4f hot_mfma(const v8sh &A, const v8sh &B, const v4f &C) {
  if constexpr (DT == TQ_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, A), __builtin_bit_cast(v8h, B), C, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, A), __builtin_bit_cast(v8bf, B), C, 0, 0,
                                                    0);
}
// The 16-bit pattern of v in the matrix type (bf16 round to nearest even,
// or f16), and what it stands for.
template <int DT>
__device__ __forceinline__ uint16_t to_mat(float v, float &back) {
  if constexpr (DT == TQ_F16) {
    const _Float16 h = (_Float16)v;
    back = (float)h;
    return __builtin_bit_cast(uint16_t, h);
  } else {
    const __bf16 h = (__bf16)v;
    back = (float)h;
    return __builtin_bit_cast(uint16_t, h);
  }
}

struct HotLds {
  float mred[4][16], lred[4][16];
  alignas(16) float ps[4][16][16];     // [wave][head][token]
  alignas(16) float accs[4][16][kHeadDim];
};

// Window chunk `item` (sequence, KV head, chunk; chunk fastest) by a
// workgroup of four waves.
template <int DT>
__device__ __attribute__((always_inline)) void hot_body(const DecodeArgs &a, HotLds &L, int item) {
  static_assert(kHotChunk == 64, "four waves of 16 tokens");
  constexpr int MT = DT == TQ_F32 ? TQ_BF16 : DT;  // matrix type of the scores
  constexpr int kEsz = DT == TQ_F32 ? 4 : 2;
  const int c = item % a.hot_parts;
  const int h = (item / a.hot_parts) % a.num_kv_heads;
  const int b = item / (a.hot_parts * a.num_kv_heads);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group;
  // the row's compressed records come first: their count needs the context
  // lengths, requested before the window's rows
  const int t0s = seq_tiles(a, lane);
  const int W = min(max(a.hot_lens[b], 0), a.hot_max);
  const int j0 = c * kHotChunk + 16 * wave;  // the wave's first token
  const int64_t tok_stride = (int64_t)a.num_kv_heads * kHeadDim;
  const uint8_t *const kb = static_cast<const uint8_t *>(a.hot_k) +
                            (((int64_t)b * a.hot_max) * tok_stride + (int64_t)h * kHeadDim) * kEsz;
  const uint8_t *const vb = static_cast<const uint8_t *>(a.hot_v) +
                            (((int64_t)b * a.hot_max) * tok_stride + (int64_t)h * kHeadDim) * kEsz;
  // tokens past the window read its last one (or token 0 of an empty window;
  // hot_max >= 1 here), and get p = 0
  const int jmax = max(W, 1) - 1;
  const int n16 = lane & 15, kg = lane >> 4;

  // the wave's V rows: lane l, coordinates 2l and 2l + 1 of each of its tokens
  float vv[16][2];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int64_t j = min(j0 + n, jmax);
    const uint8_t *row = vb + j * tok_stride * kEsz;
    if constexpr (DT == TQ_F32) {
      const float2 x = reinterpret_cast<const float2 *>(row)[lane];
      vv[n][0] = x.x;
      vv[n][1] = x.y;
    } else {
      const uint32_t x = reinterpret_cast<const uint32_t *>(row)[lane];
      vv[n][0] = hot_elem<DT>(x & 0xFFFFu);
      vv[n][1] = hot_elem<DT>(x >> 16);
    }
  }
  // the B operands: token n16's row, coordinates 32s + 8kg .. +7
  v8sh Bk[4][DT == TQ_F32 ? 3 : 1];
  {
    const int64_t j = min(j0 + n16, jmax);
    const uint8_t *row = kb + j * tok_stride * kEsz;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (DT == TQ_F32) {
        const float4 *src = reinterpret_cast<const float4 *>(row) + (32 * s + 8 * kg) / 4;
        const float4 x0 = src[0], x1 = src[1];
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // three bf16 pieces (exact for normal values)
          float back, r = xs[e];
          Bk[s][0][e] = (short)to_mat<TQ_BF16>(r, back);
          r -= back;
          Bk[s][1][e] = (short)to_mat<TQ_BF16>(r, back);
          r -= back;
          Bk[s][2][e] = (short)to_mat<TQ_BF16>(r, back);
        }
      } else {
        Bk[s][0] = *reinterpret_cast<const v8sh *>(row + 2 * (32 * s + 8 * kg));
      }
    }
  }
  // the A operands: query row n16 (head n16 of the group; zero past G),
  // coordinates 32s + 8kg .. +7, times scale log2(e), as hi + lo halves
  v8sh Ah[4], Al[4];
  {
    const float qs = a.scale * kLog2e;
    const bool live = n16 < G;
    const int64_t qrow = (int64_t)b * a.num_q_heads + (int64_t)h * G + (live ? n16 : 0);
    float xq[4][8];
    if (a.q_dtype == TQ_F32) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + qrow * kHeadDim +
                                                             32 * s + 8 * kg);
        const float4 x0 = src[0], x1 = src[1];
        xq[s][0] = x0.x; xq[s][1] = x0.y; xq[s][2] = x0.z; xq[s][3] = x0.w;
        xq[s][4] = x1.x; xq[s][5] = x1.y; xq[s][6] = x1.z; xq[s][7] = x1.w;
      }
    } else {
      const bool f16 = a.q_dtype == TQ_F16;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qrow * kHeadDim +
                                                          32 * s + 8 * kg);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t hb = (ws[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          xq[s][e] = f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)hb) : __uint_as_float(hb << 16);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = live ? qs * xq[s][e] : 0.0f;
        float back;
        Ah[s][e] = (short)to_mat<MT>(x, back);
        float back2;
        Al[s][e] = (short)to_mat<MT>(x - back, back2);
      }
  }
  v4f sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    sc = hot_mfma<MT>(Ah[s], Bk[s][0], sc);
    sc = hot_mfma<MT>(Al[s], Bk[s][0], sc);
    if constexpr (DT == TQ_F32) {
      sc = hot_mfma<MT>(Ah[s], Bk[s][1], sc);
      sc = hot_mfma<MT>(Al[s], Bk[s][1], sc);
      sc = hot_mfma<MT>(Ah[s], Bk[s][2], sc);
    }
  }
  pin_result(sc);
  // lane l, register i: head 4 kg + i, token n16 of the wave
  const bool valid = j0 + n16 < W;
  float m4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m4[i] = row_max16(valid ? sc[i] : -INFINITY);
    if (n16 == 0) L.mred[wave][4 * kg + i] = m4[i];
  }
  lds_barrier();
  float p4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = 4 * kg + i;
    const float M = fmaxf(fmaxf(L.mred[0][hd], L.mred[1][hd]), fmaxf(L.mred[2][hd], L.mred[3][hd]));
    p4[i] = valid && M != -INFINITY ? __builtin_amdgcn_exp2f(sc[i] - M) : 0.0f;
    L.ps[wave][hd][n16] = p4[i];
    const float l = row_sum16(p4[i]);
    if (n16 == 0) L.lred[wave][hd] = l;
  }
  __builtin_amdgcn_wave_barrier();
  // p v over the wave's 16 tokens for every head of the group
  float acc[16][2];
#pragma unroll
  for (int g = 0; g < 16; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    if (g < G) {  // uniform
#pragma unroll
      for (int n = 0; n < 16; n += 4) {
        const float4 pv = *reinterpret_cast<const float4 *>(&L.ps[wave][g][n]);
        acc[g][0] = fmaf(pv.x, vv[n][0], acc[g][0]);
        acc[g][1] = fmaf(pv.x, vv[n][1], acc[g][1]);
        acc[g][0] = fmaf(pv.y, vv[n + 1][0], acc[g][0]);
        acc[g][1] = fmaf(pv.y, vv[n + 1][1], acc[g][1]);
        acc[g][0] = fmaf(pv.z, vv[n + 2][0], acc[g][0]);
        acc[g][1] = fmaf(pv.z, vv[n + 2][1], acc[g][1]);
        acc[g][0] = fmaf(pv.w, vv[n + 3][0], acc[g][0]);
        acc[g][1] = fmaf(pv.w, vv[n + 3][1], acc[g][1]);
      }
      *reinterpret_cast<float2 *>(&L.accs[wave][g][2 * lane]) = make_float2(acc[g][0], acc[g][1]);
    }
  }
  lds_barrier();
  int ns;
  if (a.balanced) {
    const int per = bal_per(a, t0s);
    ns = (__builtin_amdgcn_readlane(t0s, b & 63) + per - 1) / per;
    if (a.num_seqs > 64) ns = (seq_tiles(a, b) + per - 1) / per;
  } else {
    ns = (clamped_context(a, b) + a.split_tokens - 1) / a.split_tokens;
  }
  // wave w writes the records of heads w, w + 4, ... (lane l: coordinates l, l + 64)
  const int64_t row0 = (int64_t)b * a.num_q_heads + (int64_t)h * G;  // output rows (q_len 1)
  for (int g = wave; g < G; g += 4) {  // uniform
    const float M = fmaxf(fmaxf(L.mred[0][g], L.mred[1][g]), fmaxf(L.mred[2][g], L.mred[3][g]));
    const float Ls = (L.lred[0][g] + L.lred[1][g]) + (L.lred[2][g] + L.lred[3][g]);
    float o0 = (L.accs[0][g][lane] + L.accs[1][g][lane]) + (L.accs[2][g][lane] + L.accs[3][g][lane]);
    float o1 = (L.accs[0][g][lane + 64] + L.accs[1][g][lane + 64]) + (L.accs[2][g][lane + 64] + L.accs[3][g][lane + 64]);
    wave_fwht128(o0, o1, lane);
    float *part = a.partials + ((row0 + g) * a.part_stride + ns + c) * kPartStride;
    if (lane == 0) {
      part[0] = M;
      part[1] = Ls;
    }
    part[4 + lane] = o0;
    part[68 + lane] = o1;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void hot_window_kernel(DecodeArgs a) {
  __shared__ __align__(16) HotLds L;
  hot_body<DT>(a, L, blockIdx.x);
}
__device__ __attribute__((always_inline)) void hot_body_any(const DecodeArgs &a, HotLds &L, int item) {
  if (a.hot_dtype == TQ_F32)
    hot_body<TQ_F32>(a, L, item);
  else if (a.hot_dtype == TQ_F16)
    hot_body<TQ_F16>(a, L, item);
  else
    hot_body<TQ_BF16>(a, L, item);
}

void launch_hot(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  if (a.hot_dtype == TQ_F32)
    hipLaunchKernelGGL((hot_window_kernel<TQ_F32>), grid, dim3(256), 0, stream, a);
  else if (a.hot_dtype == TQ_F16)
    hipLaunchKernelGGL((hot_window_kernel<TQ_F16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((hot_window_kernel<TQ_BF16>), grid, dim3(256), 0, stream, a);
}

// ---- 2'''. split pass on the matrix cores, one tile per wave ----------------
// The same contractions as the pass above (fp6 query digits x fp4 bit-planes for
// the scores, base-16 weight digits x fp4 value planes), arranged so that
// every wave works alone: a workgroup of 4T waves forms the query operands
// of its 4T heads once, then wave w takes tiles w, w + 4T, w + 8T, ... of
// the range, with its own online softmax and accumulators, and the waves
// meet only at the end to combine their records.  Per tile (8 pages, 128
// tokens) a wave
//   * loads the K planes and signs straight into score-operand layout (lane
//     l: token l % 16, 32 coordinates of dword l / 16 of each 16-byte token
//     record: one coalesced 256-byte load per plane and page) and the tile's
//     norms (one 16-byte piece per lane, staged in its own LDS region);
//   * scores page pairs (10 MFMAs per head tile), turns the weights of each
//     pair into base-16 digits with one exponent per (head, pair) and writes
//     them to its own LDS region in the value operand's order;
//   * loads the V planes as 16-byte pieces, lane l holding coordinates
//     8 (l % 16) .. +7 of pages 2 (l / 16) and 2 (l / 16) + 1, and
//     interleaves the two pages per coordinate in registers: register r of
//     the lane is then the B operand of coordinates 8 j + r (j = column), so
//     value MFMA r yields those coordinates and no transpose is needed;
//   * contracts the values of the tile (4 planes x 8 coordinate groups per
//     head tile) and folds the planes into 8 running sums per head tile
//     (o' = -sum_p beta_p acc_p), so its accumulators stay small.
// The K part of tile k + 4T is fetched right after tile k's scores and the V
// part right after its values, so each fetch has the other phase to arrive.
// Workgroup w of a launch runs on accelerator die (XCD) w mod 8, each with
// its own L2.  Work numbered r = 0 .. total - 1 goes to the dies in 8
// contiguous runs (die x: from ceil(x total / 8)), so neighbouring work
// shares one die's L2; item r of run x is workgroup 8 s + x, s its place in
// the run.  A grid of total + 7 workgroups covers every run.
__device__ __forceinline__ int xcd_run_start(int x, int total) { return (x * total + 7) / 8; }

// ---- stream plan (the fused decode step) -------------------------------------
// The tiles of every (sequence, KV head) group in one order (sequence-major,
// then KV head, then tile; group g = b H + h starts at C_g = H sum_{b'<b} T_b'
// + h T_b, N tiles in all).  Wave i of the split pass takes the q tiles from
// i q, q = ceil(N / (4 bal_target)) within [1, kStreamMaxTiles]: every wave
// has the same work whatever the lengths (a plan of whole ranges per group
// leaves some compute units with a third more tiles than the mean).  A
// group has R = G q_len query rows (position-major: row i G + g is head g of
// position i), in P = ceil(R / 4) head tiles of four rows; with P > 1 (5 to
// 8 heads, or a verify block) the waves go in sets of P: waves P i .. P i +
// P - 1 take the same run i of q tiles (q = ceil(P N / (4 bal_target))), one
// head tile each, side by side on one die, so the later waves' page loads
// find the first's lines in the caches and HBM serves each page once.  A run
// whose tiles span groups writes one partial record per group it touches:
// the record of (run i, group g) sits at place i + g (rows 4 u .. 4 u + 3
// from head tile u), and group g's records are the consecutive places from
// floor(C_g / q) + g to floor((C_g + T_g - 1) / q) + g.  Waves are numbered
// along the dies' runs (4 per workgroup), so a group's waves share one die.
constexpr int kStreamMaxTiles = 16;
__device__ __forceinline__ int lane_context(const DecodeArgs &a, int s) {
  return s < a.num_seqs ? clamped_context(a, s) : 0;
}
__device__ __forceinline__ int span_tiles(const DecodeArgs &a, int L) { return (L - seq_base(a, L) + 127) >> 7; }
// Tile count of sequence c0 + lane (t0: the caller's first load for lanes 0..63).
__device__ __forceinline__ int stream_block_tiles(const DecodeArgs &a, int t0, int c0, int lane) {
  return c0 == 0 ? t0 : span_tiles(a, lane_context(a, c0 + lane));
}
__device__ __forceinline__ int stream_total(const DecodeArgs &a, int t0) {
  const int lane = threadIdx.x & 63;
  int tot = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64)  // uniform
    tot += __builtin_amdgcn_readlane(wave_incl_scan_int(stream_block_tiles(a, t0, c0, lane), lane), 63);
  return tot * a.num_kv_heads;
}
// waves per run of tiles: one per head tile of the group's query rows
__device__ __forceinline__ int stream_pair(const DecodeArgs &a) { return (a.group * a.pos_count + 3) / 4; }
__device__ __forceinline__ int stream_per(const DecodeArgs &a, int N) {
  const int64_t waves = 4 * a.bal_target;
  return (int)min<int64_t>(max<int64_t>(((int64_t)stream_pair(a) * N + waves - 1) / waves, 1), kStreamMaxTiles);
}
// Per lane: sequence b, KV head h and tile t of global tile cb + min(koff +
// lane / 8, nt - 1) (a wave's slot of its run; cb, koff, nt wave-uniform,
// every tile < N) and the sequence's context length L.  Every lane of the
// wave takes part.  The eight slots' tiles are wave-uniform, so each finds
// its sequence with one ballot (the lanes j with excl_j <= c, excl not
// decreasing along the lanes), with no exchange between lanes.
__device__ __forceinline__ void stream_locate(const DecodeArgs &a, int t0, int L0, int cb, int koff, int nt, int &b,
                                              int &h, int &t, int &L) {
  const int lane = threadIdx.x & 63, H = a.num_kv_heads, mine = lane >> 3;
  int run = 0, sc = 0, se = 0, sT = 1;
  b = L = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {  // uniform
    const int Ll = c0 == 0 ? L0 : lane_context(a, c0 + lane);
    const int T = c0 == 0 ? t0 : span_tiles(a, Ll);
    const int incl = wave_incl_scan_int(H * T, lane) + run;
    const int excl = incl - H * T;
    const int end = __builtin_amdgcn_readlane(incl, 63);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = cb + min(koff + k, nt - 1);  // uniform
      if (c >= run && c < end) {  // uniform: slot k's tile lies in this block (then T_j > 0)
        const int j = __builtin_popcountll(__ballot(excl <= c)) - 1;
        const int ej = __builtin_amdgcn_readlane(excl, j), Tj = __builtin_amdgcn_readlane(T, j);
        const int Lj = __builtin_amdgcn_readlane(Ll, j);
        if (mine == k) {
          b = c0 + j;
          L = Lj;
          sc = c;
          se = ej;
          sT = Tj;
        }
      }
    }
    run = end;
  }
  const int rel = sc - se;
  h = rel / sT;
  t = rel - h * sT;
}
// Exclusive prefix P_b = H sum_{b'<b} T_b' and T_b of sequence b (uniform b).
__device__ __forceinline__ void stream_prefix(const DecodeArgs &a, int t0, int b, int &P, int &Tb) {
  const int lane = threadIdx.x & 63, H = a.num_kv_heads;
  int run = 0;
  P = Tb = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {  // uniform
    const int T = stream_block_tiles(a, t0, c0, lane);
    const int incl = wave_incl_scan_int(H * T, lane) + run;
    if (b >= c0 && b < c0 + 64) {  // uniform
      Tb = __builtin_amdgcn_readlane(T, b - c0);
      P = __builtin_amdgcn_readlane(incl, b - c0) - H * Tb;
    }
    run = __builtin_amdgcn_readlane(incl, 63);
  }
}

// The descriptor of wave `wave` of workgroup `blk` of the split pass's grid
// (all lanes of one wave call this): its run of tiles on the stream plan,
// the block ids of its tile slots (as the split pass loads pages: lane l
// holds page l % 8 of slot l / 8 in ids0 and of slot 8 + l / 8 in ids1; a
// page past the keys re-reads its tile's first page, a slot past the wave's
// last tile repeats that tile) and the slots' (sequence, KV head, tile,
// length).  Words: [0, 64) ids0, [64, 128) ids1, [128, 192) the 16 slots,
// [192, 196) (tiles, run, head tile, 0); tiles 0: no work for the wave.
__device__ __forceinline__ void stream_describe(const DecodeArgs &a, int blk, int wave) {
  const int lane = threadIdx.x & 63;
  const int Lw = lane_context(a, lane);
  const int t0s = span_tiles(a, Lw);
  const int N = stream_total(a, t0s);
  const int q = stream_per(a, N);
  const int P = stream_pair(a);
  const int nwg = (P * ((N + q - 1) / q) + 3) >> 2;
  const int x = blk & 7, rpos = xcd_run_start(x, nwg) + (blk >> 3);
  int ntiles = 0, iw = 0, ut = 0;
  if (rpos < xcd_run_start(x + 1, nwg)) {  // uniform
    iw = (4 * rpos + wave) / P;
    ut = (4 * rpos + wave) - iw * P;
    ntiles = max(min(q, N - iw * q), 0);
  }
  uint32_t *d = a.desc + ((int64_t)blk * 4 + wave) * kDescWords;
  if (ntiles > 0) {  // uniform
    const int e = lane & 7;
    auto slot_ids = [&](int koff) __attribute__((always_inline)) {
      int sb, sh, st, sl;
      stream_locate(a, t0s, Lw, iw * q, koff, ntiles, sb, sh, st, sl);
      const int tile0 = seq_base(a, sl) + 128 * st, tok = tile0 + 16 * e;
      if (e == 0) reinterpret_cast<int4 *>(d + 128)[koff + (lane >> 3)] = make_int4(sb, sh, st, sl);
      const int id = a.block_tables[(int64_t)sb * a.max_blocks + page_entry(a, (tok < sl ? tok : tile0) >> 4)];
      return id * a.num_kv_heads + sh;
    };
    d[lane] = (uint32_t)slot_ids(0);
    d[64 + lane] = (uint32_t)slot_ids(8);
  }
  if (lane == 0) *reinterpret_cast<int4 *>(d + 192) = make_int4(ntiles, iw, ut, 0);
  // the merge's view of groups blk * 4 + wave, + 4 grid, ...: group g = (b,
  // h)'s records are the places floor(C_g / q) + g .. floor((C_g + T_b - 1)
  // / q) + g (no record when T_b = 0)
  for (int g = blk * 4 + wave; g < a.num_seqs * a.num_kv_heads; g += 4 * a.bal_grid) {  // uniform
    const int b = g / a.num_kv_heads, h = g - b * a.num_kv_heads;
    int Pb, Tb;
    stream_prefix(a, t0s, b, Pb, Tb);
    const int c0 = Pb + h * Tb, i0 = c0 / q;
    if (lane == 0) a.ginfo[g] = make_int2(i0 + g, Tb > 0 ? (c0 + Tb - 1) / q - i0 + 1 : 0);
  }
}

// One reference R per head serves the scores and the accumulators: it moves
// (rarely) when a score exceeds it by 2^64, and the digits of a pair carry
// the R they were formed with.
// 128 digits of one A row, padded to 68 dwords: the rows of the four heads a
// wave writes together (4 rows apart) start 16 banks apart
constexpr int kWqRowW = 136;
template <int T>
struct WaveLds {
  union {
    QPrepLds<T> q;  // start-up scratch of the query operands
    struct {
      alignas(16) uint16_t wq[4 * T][T][16][kWqRowW];  // per wave: [head tile][head*4+digit][K slot]
      alignas(16) uint32_t nrm[4 * T][64][4];         // per wave: the tile's norms, 16 bytes per lane
      int2 stats[4 * T][T][4][4];                      // per wave: [head tile][head][pair]: (exponent field, R bits)
    } w;
    struct {
      float acc[4 * T][4 * T][kHeadDim];  // [wave][head][coordinate]
      float m[4 * T][4 * T], l[4 * T][4 * T];
    } red;
  };
};

template <int T>
union WaveOrHotLds {
  WaveLds<T> w;
  HotLds h;
};

// Workgroups past the plan's grid take the exact window's chunks (a call
// with a hot window, T = 1): they run beside the split pass instead of after it.
// STREAM: the fused decode step's pass, on the stream plan above, with the
// query operands formed beforehand (one head tile; each wave on its own).
template <int T, bool STREAM>
__global__ __launch_bounds__(256 * T, T == 1 ? 2 : 1) void split_wave_kernel(DecodeArgs a) {
  static_assert(!STREAM || T == 1, "the stream plan serves one head tile");
  constexpr int NW = 4 * T;
  __shared__ __align__(16) WaveOrHotLds<T> smu;
  // stream plan: (sequence, KV head, tile, context length) of each tile slot of a wave
  __shared__ int4 slot_sh[STREAM ? 4 : 1][kStreamMaxTiles];
  if constexpr (T == 1 && !STREAM) {
    if ((int)blockIdx.x >= a.bal_grid) {  // uniform
      hot_body_any(a, smu.h, (int)blockIdx.x - a.bal_grid);
      return;
    }
  }
  WaveLds<T> &sm = smu.w;
  constexpr bool kProjAll = T == 1;
  QPrepRegs<true> qpr;
  QPrepRegs<false> qpn;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t16 = lane & 15, grow = lane >> 4;
  const int qlen = a.q_len - a.pos0, nrows = a.group * a.pos_count, G = a.group;
  // the range (ranges plan) or the wave's current group (stream plan): its
  // sequence b, KV head h, keys [s0, s1) and the sequence's length L
  int b, h, L, s0, s1, ntiles, jr = 0;
  int iw = 0;  // stream plan: the wave's run of tiles in the order
  int ut = 0;  // stream plan: the wave's head tile (query rows 4 ut .. 4 ut + 3 of the group)
  // block ids of this wave's tile slots (at most 16) as (block id) x (KV
  // heads) + KV head: lane l holds page l % 8 of slot l / 8 (ids0) and of
  // slot 8 + l / 8 (ids1); a page past the keys re-reads its tile's first
  // page, and a slot past the wave's last tile repeats that tile (the tokens
  // are masked)
  int ids0, ids1;
  if constexpr (STREAM) {
    // the wave's descriptor, formed by the operands launch: every load at
    // once (the descriptor exists for every wave of the grid)
    const uint32_t *d = a.desc + ((int64_t)blockIdx.x * 4 + wave) * kDescWords;
    const int4 meta = *reinterpret_cast<const int4 *>(d + 192);
    ids0 = (int)d[lane];
    ids1 = (int)d[64 + lane];
    const int4 sl = reinterpret_cast<const int4 *>(d + 128)[lane & 15];
    ntiles = __builtin_amdgcn_readfirstlane(meta.x);
    if (ntiles <= 0) return;  // uniform: no run for this wave (this plan has no workgroup barrier)
    iw = __builtin_amdgcn_readfirstlane(meta.y);
    ut = __builtin_amdgcn_readfirstlane(meta.z);
    if (lane < kStreamMaxTiles) slot_sh[wave][lane] = sl;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const int4 f0 = slot_sh[wave][0];
    b = __builtin_amdgcn_readfirstlane(f0.x);
    h = __builtin_amdgcn_readfirstlane(f0.y);
    L = __builtin_amdgcn_readfirstlane(f0.w);
    s0 = seq_base(a, L);
    s1 = L;
  } else {
    // the context lengths (the plan needs them first), then the projection
    // operands, which do not depend on the plan (loads return in order: the
    // plan then waits for the lengths only)
    const int t0s = seq_tiles(a, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (kProjAll || wave < 4) qprep_load_sh<true>(a, wave, lane, qpr);  // uniform
    __builtin_amdgcn_sched_barrier(0);
    const int per = bal_per(a, t0s);
    int Tb;
    bal_locate(a, t0s, per, blockIdx.x, b, h, jr, Tb);
    if (b >= a.num_seqs) return;  // uniform: past the last range
    L = clamped_context(a, b);
    const int base = seq_base(a, L);
    s0 = base + 128 * per * jr;
    s1 = min(base + 128 * per * (jr + 1), L);
    ntiles = (s1 - s0 + 127) >> 7;
    const int32_t *btab = a.block_tables + (int64_t)b * a.max_blocks;
    const int e = lane & 7;
    int k = wave + NW * (lane >> 3);
    int tile0 = s0 + 128 * min(k, ntiles - 1);
    int tok = tile0 + 16 * e;
    ids0 = btab[page_entry(a, (tok < s1 ? tok : tile0) >> 4)] * a.num_kv_heads + h;
    k += 8 * NW;
    tile0 = s0 + 128 * min(k, ntiles - 1);
    tok = tile0 + 16 * e;
    ids1 = btab[page_entry(a, (tok < s1 ? tok : tile0) >> 4)] * a.num_kv_heads + h;
  }
  int64_t grp = (int64_t)b * a.num_kv_heads + h;
  const int pair = STREAM ? stream_pair(a) : 1;
  auto page_id = [&](int slot, int e) __attribute__((always_inline)) {
    const int src = slot < 8 ? ids0 : ids1;
    return __builtin_amdgcn_readlane(src, 8 * (slot & 7) + e);
  };

  // the precomputed operands (stream plan): kQopsDwords per lane as 16-byte pieces
  u32x4 qo[kQopsDwords / 4];
  auto load_qops = [&]() __attribute__((always_inline)) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.qops) + (grp * pair + ut) * (kQopsDwords / 4) * 64 + lane;
#pragma unroll
    for (int c = 0; c < kQopsDwords / 4; ++c) qo[c] = src[c * 64];
  };
  if constexpr (STREAM) {
    load_qops();
  } else if (kProjAll || wave < 4) {  // uniform
    qprep_load_q<true>(a, grp, wave, lane, qpr);
  } else {
    qprep_load_q<false>(a, grp, wave, lane, qpn);
  }

  float beta[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) beta[p] = uniform(a.cb.beta[p]);
  const BSplitK bk = bsplit_consts();
  const uint32_t nib = in_vgpr(0x000F000Fu);
  const uint32_t s80 = in_vgpr((t16 & 3) == 3 ? 0u : 0x80008000u);
  const int kap0 = 8 * (t16 & 3) + (t16 >> 2);
  const int gA = t16 >> 2, rA = lane & 3;
  const uint8_t *const kc = a.k_cache, *const vc = a.v_cache;
  // the lane's K record: coordinate chunk grow, token t16 (planes 0..2, signs)
  const uint32_t ko = (uint32_t)k_record(grow, t16);
  // norms: lanes 0..31 K page l / 4 at 1024 + 16 (l % 4) (n_k, gamma), lanes
  // 32..47 V page (l - 32) / 2 at 768 + 16 (l % 2), lanes 48..63 repeat 32..47
  const int ne = lane < 32 ? lane >> 2 : ((lane - 32) & 15) >> 1;
  const uint32_t no = lane < 32 ? 1024u + 16u * (uint32_t)(lane & 3) : 768u + 16u * (uint32_t)(lane & 1);
  const bool nk = lane < 32;

  // per-wave state (lane: head grow of tile u)
  float R[T], lsum[T];
  float tot[T][8];
  v4f corr[T];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    R[u] = -INFINITY;
    lsum[u] = 0.0f;
    corr[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 8; ++r) tot[u][r] = 0.0f;
  }

  u32x4 KP[8];
  u32x4 NR;
  u32x4 VA[3][2];
  // fetches of tile slot i (unconditional: past the wave's last tile they
  // repeat its own pages, which are valid)
  auto load_k = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint8_t *kp = uniform_ptr(kc + (int64_t)page_id(i, e) * kKPage);
      KP[e] = load_at<u32x4>(kp, ko);
    }
    const int64_t pid = (int64_t)__builtin_amdgcn_ds_bpermute(4 * (8 * (i & 7) + ne), i < 8 ? ids0 : ids1);
    const uint8_t *np = nk ? kc + pid * kKPage : vc + pid * kVPage;
    NR = *reinterpret_cast<const u32x4 *>(np + no);
  };
  auto load_v = [&](int i) __attribute__((always_inline)) {
    const int src = i < 8 ? ids0 : ids1;
    const int pa = __builtin_amdgcn_ds_bpermute(4 * (8 * (i & 7) + 2 * grow), src);
    const int pb = __builtin_amdgcn_ds_bpermute(4 * (8 * (i & 7) + 2 * grow + 1), src);
    const uint8_t *va = vc + (int64_t)pa * kVPage + 16 * t16;
    const uint8_t *vb = vc + (int64_t)pb * kVPage + 16 * t16;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      VA[p][0] = *reinterpret_cast<const u32x4 *>(va + kVPlane * p);
      VA[p][1] = *reinterpret_cast<const u32x4 *>(vb + kVPlane * p);
    }
  };

  int slot = 0;
  // tile k of the range (wave w: w, w + NW, ...) or of the wave's own tiles
  constexpr int kStep = STREAM ? 1 : NW;
  int k = STREAM ? 0 : wave;
  // the first tile's pages are requested before the query operands are
  // formed, so that their memory latency overlaps that work
  if (k < ntiles) {  // uniform
    load_k(0);
    load_v(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // query operands of all head tiles (every wave scores)
  v8i Aq[T][5];
  int scq[T][5];
  v4f cinit[T], qinit[T];
  int tiles_all[T];
#pragma unroll
  for (int u = 0; u < T; ++u) tiles_all[u] = u;
  auto set_qops = [&]() __attribute__((always_inline)) {
    const auto wd = [&](int i) __attribute__((always_inline)) { return qo[i >> 2][i & 3]; };
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      Aq[0][p] = v8i{(int)wd(6 * p), (int)wd(6 * p + 1), (int)wd(6 * p + 2), (int)wd(6 * p + 3), (int)wd(6 * p + 4),
                     (int)wd(6 * p + 5), 0, 0};
      scq[0][p] = (int)wd(30 + p);
    }
    cinit[0] = v4f{__uint_as_float(wd(35)), __uint_as_float(wd(36)), __uint_as_float(wd(37)), __uint_as_float(wd(38))};
    qinit[0] = v4f{__uint_as_float(wd(39)), __uint_as_float(wd(40)), __uint_as_float(wd(41)), __uint_as_float(wd(42))};
  };
  if constexpr (STREAM) {
    set_qops();
  } else if (kProjAll || wave < 4) {  // uniform
    qprep_compute<T, T, true, true>(a, sm.q, qpr, tid, wave, tiles_all, Aq, scq, cinit, qinit);
  } else {
    qprep_compute<T, T, true, false>(a, sm.q, qpn, tid, wave, tiles_all, Aq, scq, cinit, qinit);
  }
  uint32_t *const nrm = &sm.w.nrm[wave][0][0];
  const uint16_t *const nh = reinterpret_cast<const uint16_t *>(nrm);
  // the last key each of the lane's rows sees (causal over a verify block)
  int lim[T], low[T];
  auto set_lims = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const int hi = L - qlen + (4 * (u + ut) + grow) / G + 1;
      lim[u] = min(s1, hi);
      low[u] = window_low(a, hi);
    }
  };
  set_lims();
  const float bsum = (beta[0] + beta[1]) + (beta[2] + beta[3]);
  // stream plan: the wave's record of its current group (place iw + group,
  // the rows of its head tile)
  auto write_record = [&]() __attribute__((always_inline)) {
    // keep the matrix ops out of the per-head branch below
    asm volatile("" : "+v"(corr[0]));
#pragma unroll
    for (int r = 0; r < 8; ++r) asm volatile("" : "+v"(tot[0][r]));
    const float cs = (corr[0][0] + corr[0][1]) + (corr[0][2] + corr[0][3]);
    const float ls = row_sum16(lsum[0]);
    if (4 * ut + grow < nrows) {
      float *part = a.partials + (((int64_t)iw + grp) * nrows + 4 * ut + grow) * kPartStride;
      if (t16 == 0) {
        part[0] = R[0];
        part[1] = ls;
      }
      float4 *o4 = reinterpret_cast<float4 *>(part + 4 + 8 * t16);
      o4[0] = make_float4(tot[0][0] - bsum * cs, tot[0][1] - bsum * cs, tot[0][2] - bsum * cs, tot[0][3] - bsum * cs);
      o4[1] = make_float4(tot[0][4] - bsum * cs, tot[0][5] - bsum * cs, tot[0][6] - bsum * cs, tot[0][7] - bsum * cs);
    }
  };
  for (; k < ntiles; k += kStep, ++slot) {  // uniform per wave
    const int nslot = k + kStep < ntiles ? slot + 1 : slot;
    int tok0;
    if constexpr (STREAM) {
      const int4 si = slot_sh[wave][slot];
      const int st = __builtin_amdgcn_readfirstlane(si.z);
      if (slot > 0 && st == 0) {  // uniform: the wave's next group starts here
        write_record();
        b = __builtin_amdgcn_readfirstlane(si.x);
        h = __builtin_amdgcn_readfirstlane(si.y);
        L = __builtin_amdgcn_readfirstlane(si.w);
        grp = (int64_t)b * a.num_kv_heads + h;
        s0 = seq_base(a, L);
        s1 = L;
        load_qops();
        set_qops();
        set_lims();
        R[0] = -INFINITY;
        lsum[0] = 0.0f;
        corr[0] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < 8; ++r) tot[0][r] = 0.0f;
      }
      tok0 = s0 + 128 * st;
    } else {
      tok0 = s0 + 128 * k;
    }
    // ---- raw scores of the tile's 8 pages (log2 units) ------------------------
    // K page e: n_k at halves 32 e + t, gamma at 32 e + 16 + t; V page e: 256 + 16 e + t
    *reinterpret_cast<u32x4 *>(nrm + 4 * lane) = NR;
    float rs[T][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float nkv = half_lo(nh[32 * e + t16]), gmv = half_lo(nh[32 * e + 16 + t16]);
      const uint32_t w0 = KP[e][0], w1 = KP[e][1], w2 = KP[e][2], w3 = KP[e][kKSignField];
      const v8i B0 = bsplit(w0, bk), B1 = bsplit(w1, bk), B2 = bsplit(w2, bk);
      const v8i Bx = bsplit(w0 ^ w1 ^ w2, bk), Bs = bsplit(w3, bk);
      const int tq = tok0 + 16 * e + t16;
#pragma unroll
      for (int u = 0; u < T; ++u) {
        v4f c = mfma_f6f4(Aq[u][0], B0, cinit[u], scq[u][0]);
        c = mfma_f6f4(Aq[u][1], B1, c, scq[u][1]);
        c = mfma_f6f4(Aq[u][2], B2, c, scq[u][2]);
        c = mfma_f6f4(Aq[u][3], Bx, c, scq[u][3]);
        v4f qv = mfma_f6f4(Aq[u][4], Bs, qinit[u], scq[u][4]);
        pin_result(c);
        pin_result(qv);
        const float inner = fmaf(gmv, (qv[0] + qv[1]) + (qv[2] + qv[3]), (c[0] + c[1]) + (c[2] + c[3]));
        // a slot the lane's row does not see (past the range, or causal) is -inf
        rs[u][e] = tq < lim[u] && tq >= low[u] ? nkv * inner : -INFINITY;
      }
    }
    // the K part of the next tile (the last tile re-reads its own), issued as
    // soon as this tile's K registers are consumed: scheduling barriers keep
    // the compiler from sinking the loads to their use, which would expose
    // the whole memory latency
    __builtin_amdgcn_sched_barrier(0);
    load_k(nslot);
    __builtin_amdgcn_sched_barrier(0);
    // ---- the head's reference moves when a score exceeds it by 2^64 (or it is
    // still -inf); the lanes of a head move together
#pragma unroll
    for (int u = 0; u < T; ++u) {
      float mx = rs[u][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, rs[u][e]);
      if (__builtin_amdgcn_ballot_w64(mx > R[u] + (float)kRefStep)) {  // uniform, rare
        const float nr = fmaxf(R[u], ceilf(row_max16(mx)));
        if (nr > R[u]) {
          const float f = R[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(R[u] - nr);
          lsum[u] *= f;
          corr[u] *= f;
#pragma unroll
          for (int r = 0; r < 8; ++r) tot[u][r] *= f;
          R[u] = nr;
        }
      }
    }
    // ---- weights of the 4 page pairs as base-16 digits -------------------------
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float nv0 = half_lo(nh[256 + 32 * q + t16]), nv1 = half_lo(nh[256 + 32 * q + 16 + t16]);
#pragma unroll
      for (int u = 0; u < T; ++u) {
        const float r0 = rs[u][2 * q], r1 = rs[u][2 * q + 1];
        // (R stays -inf while the head has seen no key: select, never -inf - -inf)
        const float p0 = r0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(r0 - R[u]);
        const float p1 = r1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(r1 - R[u]);
        lsum[u] += p0 + p1;
        // a slot past the visible range may hold any norm bits (Inf, NaN)
        const float w0 = r0 == -INFINITY ? 0.0f : p0 * nv0;
        const float w1 = r1 == -INFINITY ? 0.0f : p1 * nv1;
        const int mk = row_max16_nonneg(max(__float_as_int(w0), __float_as_int(w1)));  // w >= 0
        const uint32_t exb = max((uint32_t)mk & 0x7F800000u, 14u << 23);
        const float mult = __uint_as_float(0x86000000u - exb);  // 2^(141 - ex)
        const uint32_t X0 = __float_as_uint(fmaf(w0, mult, 8388608.0f));
        const uint32_t X1 = __float_as_uint(fmaf(w1, mult, 8388608.0f));
        const uint32_t XX = __builtin_amdgcn_perm(X1, X0, 0x05040100u);  // X0 lo16 | X1 lo16 << 16
        uint16_t *wr = &sm.w.wq[wave][u][4 * grow][32 * q + kap0];
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // digit r (place 16^(3-r)) of both tokens, with the slot's sign
          const uint32_t D = ((XX >> (12 - 4 * r)) & nib) | s80;
          wr[r * kWqRowW] = (uint16_t)D;
          wr[r * kWqRowW + 4] = (uint16_t)(D >> 16);
        }
        sm.w.stats[wave][u][grow][q] = make_int2((int)(exb >> 23), __float_as_int(R[u]));
      }
    }
    // ---- values of the tile --------------------------------------------------
    v8i Aw[T];
    int sw[T];
#pragma unroll
    for (int u = 0; u < T; ++u) {
      Aw[u] = fp6_operand(&sm.w.wq[wave][u][t16][32 * grow], 0x1p-21f);  // d 2^-24 -> d/8 (row: 272 bytes)
      const int2 st = sm.w.stats[wave][u][gA][grow];
      const float ra = __shfl(R[u], 16 * gA, 64);  // R of head gA now
      const float d = fmaxf(__int_as_float(st.y) - ra, -300.0f);  // NaN (both -inf) -> -300
      sw[u] = min(max(st.x + 1 - 4 * rA + (int)d, 0), 254);  // E8M0 of 2^(ex-126-4r+R_pair-R)
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t W[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)  // coordinate 8 t16 + r of both pages: page a low, page b high
        W[p] = __builtin_amdgcn_perm(VA[p][1][r >> 1], VA[p][0][r >> 1], (r & 1) ? 0x07060302u : 0x05040100u);
      const v8i V0 = bsplit(W[0], bk), V1 = bsplit(W[1], bk), V2 = bsplit(W[2], bk);
      const v8i Vx = bsplit(W[0] ^ W[1] ^ W[2], bk);
#pragma unroll
      for (int u = 0; u < T; ++u) {
        const v4f z = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const v4f c0 = mfma_f6f4(Aw[u], V0, z, sw[u]);
        const v4f c1 = mfma_f6f4(Aw[u], V1, z, sw[u]);
        const v4f c2 = mfma_f6f4(Aw[u], V2, z, sw[u]);
        const v4f c3 = mfma_f6f4(Aw[u], Vx, z, sw[u]);
        float o = tot[u][r];
        o = fmaf(-beta[0], (c0[0] + c0[1]) + (c0[2] + c0[3]), o);
        o = fmaf(-beta[1], (c1[0] + c1[1]) + (c1[2] + c1[3]), o);
        o = fmaf(-beta[2], (c2[0] + c2[1]) + (c2[2] + c2[3]), o);
        tot[u][r] = fmaf(-beta[3], (c3[0] + c3[1]) + (c3[2] + c3[3]), o);
      }
    }
    {
      const v8i C1 = v8i{(int)0xEEEEEEEEu, (int)0xDDDDDDDDu, (int)0xAAAAAAAAu, 0, 0, 0, 0, 0};
      const v8i C2 = v8i{(int)0xAAAAAAAAu, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < T; ++u) {
        corr[u] = mfma_f6f4(Aw[u], C1, corr[u], sw[u]);
        corr[u] = mfma_f6f4(Aw[u], C2, corr[u], sw[u]);
      }
    }
    // the V part of the next tile
    __builtin_amdgcn_sched_barrier(0);
    load_v(nslot);
    __builtin_amdgcn_sched_barrier(0);
  }
  // keep the matrix ops out of the per-head branches below
#pragma unroll
  for (int u = 0; u < T; ++u) {
    asm volatile("" : "+v"(corr[u]));
#pragma unroll
    for (int r = 0; r < 8; ++r) asm volatile("" : "+v"(tot[u][r]));
  }

  if constexpr (STREAM) {
    write_record();
    return;
  }
  // ---- the waves combine their records -----------------------------------------
  lds_barrier();  // every wave is done with its LDS region
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const int hd = 4 * u + grow;
    const float cs = (corr[u][0] + corr[u][1]) + (corr[u][2] + corr[u][3]);
#pragma unroll
    for (int r = 0; r < 8; ++r) sm.red.acc[wave][hd][8 * t16 + r] = tot[u][r] - bsum * cs;
    const float ls = row_sum16(lsum[u]);
    if (t16 == 0) {
      sm.red.m[wave][hd] = R[u];
      sm.red.l[wave][hd] = ls;
    }
  }
  lds_barrier();
  // wave w writes the record of head w
  if (wave < nrows) {  // uniform
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, sm.red.m[v][wave]);
    float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float mv = sm.red.m[v][wave];
      const float f = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
      l = fmaf(f, sm.red.l[v][wave], l);
      o0 = fmaf(f, sm.red.acc[v][wave][lane], o0);
      o1 = fmaf(f, sm.red.acc[v][wave][lane + 64], o1);
    }
    float *part = a.partials + (query_out_row(a, grp, wave) * a.part_stride + jr) * kPartStride;
    if (lane == 0) {
      part[0] = M;
      part[1] = l;
    }
    part[4 + lane] = o0;
    part[68 + lane] = o1;
  }
}

// ---- 0. fused decode step: the append and the query operands ----------------
// A decode step appends each sequence's new token and then attends over the
// whole cache.  The append is a short, latency-bound launch; this one also
// does the split pass's query set-up, which depends only on (sequence, KV
// head): workgroups past the append's form one group's query operands each
// (the same code as the split pass's prologue) and store them.  The split
// pass (stream plan) then loads a group's operands where a wave starts on it.
union StepLds {
  QPrepLds<1> q;
  float rsh[kAppendWaves][kHeadDim];
};

template <int DT>
__global__ __launch_bounds__(256, 2) void step_prep_kernel(EncodeArgs ea, DecodeArgs a, int n_append, int n_items) {
  __shared__ __align__(16) StepLds sm;
  const int wg = blockIdx.x;
  if (wg < n_append) {  // uniform
    append_body<DT, 3>(ea, sm.rsh, wg);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wg >= n_append + n_items) {  // uniform: the descriptors of split workgroup wg - n_append - n_items
    stream_describe(a, wg - n_append - n_items, wave);
    return;
  }
  // item: (group, head tile), the stream plan's pair factor of them per group
  const int64_t item = wg - n_append;
  const int P = stream_pair(a);
  const int64_t grp = item / P;
  const int hbase = 4 * (int)(item - grp * P);
  QPrepRegs<true> qpr;
  qprep_load_sh<true>(a, wave, lane, qpr);
  qprep_load_q<true>(a, grp, wave, lane, qpr, hbase);
  __builtin_amdgcn_sched_barrier(0);
  v8i Aq[1][5];
  int scq[1][5];
  v4f ci[1], qi[1];
  const int tiles[1] = {0};
  qprep_compute<1, 1, true, true, false>(a, sm.q, qpr, tid, wave, tiles, Aq, scq, ci, qi, hbase);
  if (wave == 0) {
    uint32_t w[kQopsDwords];
#pragma unroll
    for (int p = 0; p < 5; ++p) {
#pragma unroll
      for (int i = 0; i < 6; ++i) w[6 * p + i] = (uint32_t)Aq[0][p][i];
      w[30 + p] = (uint32_t)scq[0][p];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[35 + i] = __float_as_uint(ci[0][i]);
      w[39 + i] = __float_as_uint(qi[0][i]);
    }
    w[43] = 0u;
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.qops) + item * (kQopsDwords / 4) * 64 + lane;
#pragma unroll
    for (int c = 0; c < kQopsDwords / 4; ++c) dst[c * 64] = u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
  }
}

// ---- 3. merge ---------------------------------------------------------------
// LSE combine of the chunk partials of an output row, o' = acc'/l, one
// inverse FWHT, store.  W waves share a row (4/W rows per workgroup); wave w
// of a row takes chunks NB w .. NB w + NB - 1, then NB (w + W) .., and issues
// every load of a batch of NB (16, or 32 for the stream plan's rows of up to
// about a hundred records) together, so up to NB W chunks cost one memory
// round trip.  Lane l owns coordinates l and l + 64, lane e < NB the
// statistics of chunk e of the batch.  The waves of a row then meet in LDS.
constexpr int kMergeBatch = 16;

template <int W, int NB = kMergeBatch>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int64_t rows) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave % W;
  const int64_t r = (int64_t)blockIdx.x * (4 / W) + wave / W;
  __shared__ float wm[4], wl[4];
  __shared__ float wa[4][kHeadDim];
  int ns = 0;
  const float *part = a.partials;
  int64_t rstride = kPartStride;  // floats from one record of the row to the next
  if (r < rows) {
    const int64_t per_seq = (int64_t)a.q_len * a.num_q_heads;
    const int b = (int)(r / per_seq);
    const int t = (int)((r / a.num_q_heads) % a.q_len);
    if (a.balanced == 2) {  // stream plan: the group's records are consecutive places
      const int hq = (int)(r % a.num_q_heads), h = hq / a.group, hd = t * a.group + hq - h * a.group;
      const int nrows = a.group * a.q_len;
      // the group's first place and record count, from the operands launch
      const int2 gi = a.ginfo[(int64_t)b * a.num_kv_heads + h];
      ns = __builtin_amdgcn_readfirstlane(gi.y);
      part += ((int64_t)__builtin_amdgcn_readfirstlane(gi.x) * nrows + hd) * kPartStride;
      rstride = (int64_t)nrows * kPartStride;
    } else {
      if (a.balanced) {
        const int per = bal_per(a, seq_tiles(a, lane));
        ns = (seq_tiles(a, b) + per - 1) / per;
      } else {
        const int L = clamped_context(a, b);
        const int vis = max(0, L - seq_base(a, L) - a.q_len + t + 1);
        ns = (vis + a.split_tokens - 1) / a.split_tokens;
      }
      ns += a.hot_parts;  // the window's records follow
      part += r * a.part_stride * kPartStride;
    }
  }
  float M = -INFINITY, Ls = 0.0f, A0 = 0.0f, A1 = 0.0f;  // Ls: lanes < 16, per chunk slot
  for (int base = NB * wr; base < ns; base += NB * W) {  // uniform
    float v0[NB], v1[NB];
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      const float *p = part + (int64_t)min(base + e, ns - 1) * rstride;
      v0[e] = p[4 + lane];
      v1[e] = p[68 + lane];
    }
    const bool live = lane < NB && base + lane < ns;
    const float *ps = part + (int64_t)min(base + (lane & (NB - 1)), ns - 1) * rstride;
    const float m0 = ps[0], l = ps[1];  // unconditional loads
    const float m = live ? m0 : -INFINITY;
    const float mb = wave_max(m);
    if (mb > M) {  // uniform: move the wave's reference (nothing to rescale while it is -inf)
      const float c = M == -INFINITY ? 0.0f : exp2f(M - mb);
      Ls *= c;
      A0 *= c;
      A1 *= c;
      M = mb;
    }
    const float f = m == -INFINITY ? 0.0f : exp2f(m - M);
    Ls = fmaf(f, live ? l : 0.0f, Ls);
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      const float fe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), e));  // 0 past ns
      A0 = fmaf(fe, v0[e], A0);
      A1 = fmaf(fe, v1[e], A1);
    }
  }
  const float Lw = wave_sum(Ls);
  if (W > 1) {
    if (lane == 0) {
      wm[wave] = M;
      wl[wave] = Lw;
    }
    wa[wave][lane] = A0;
    wa[wave][64 + lane] = A1;
    lds_barrier();
  }
  if (wr != 0 || r >= rows) return;
  float Mx = M;
#pragma unroll
  for (int w = 1; w < W; ++w) Mx = fmaxf(Mx, wm[wave + w]);
  float Lt = 0.0f, o0 = 0.0f, o1 = 0.0f;
  if (W == 1) {
    Lt = Lw;
    o0 = A0;
    o1 = A1;
  } else {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = wm[wave + w];
      const float c = mw == -INFINITY ? 0.0f : exp2f(mw - Mx);
      Lt = fmaf(c, wl[wave + w], Lt);
      o0 = fmaf(c, wa[wave + w][lane], o0);
      o1 = fmaf(c, wa[wave + w][64 + lane], o1);
    }
  }
  if (Lt > 0.0f) {
    const float inv = 1.0f / Lt;
    o0 *= inv;
    o1 *= inv;
  } else {  // no visible key
    o0 = 0.0f;
    o1 = 0.0f;
  }
  wave_fwht128(o0, o1, lane);
  store_from_float(a.out, a.out_dtype, r * kHeadDim + lane, o0);
  store_from_float(a.out, a.out_dtype, r * kHeadDim + 64 + lane, o1);
}

template <int G>
hipError_t launch_split(const DecodeArgs &a, hipStream_t stream) {
  dim3 grid((unsigned)(a.num_seqs * a.q_len), (unsigned)a.num_kv_heads, (unsigned)a.num_splits);
  switch (a.cb.bits) {
    case 2: hipLaunchKernelGGL((split_valu_kernel<G, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((split_valu_kernel<G, 3>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((split_valu_kernel<G, 4>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// ---- device scratch of the no-allocation decode call ------------------------
// In host code `scratch` names a host-side stand-in, never the device array:
// its device address comes only from hipGetSymbolAddress, once per device
// with that device current, and every launch takes that address.  Calls of
// tq_decode_attention_noalloc on one device share the array: overlapping
// calls (several streams, several threads) race.  Nothing in it needs to
// start at zero: the split passes write every partial record the merge reads.
namespace {
__device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  if (ptr) *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Kernels templated on the group size are built for 1, 2, 4, 8 and 16
// heads; another size runs on the next one up.
static int group_capacity(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : g <= 16 ? 16 : 0; }

hipError_t launch_step_prep(const EncodeArgs *ea, const DecodeArgs &a, hipStream_t stream) {
  // no append (ea null): the query operands of a verify block only
  const int64_t vectors = ea ? ea->num_tokens * ea->num_kv_heads : 0;
  const int n_append = (int)((vectors + kAppendWaves - 1) / kAppendWaves);
  // one operands workgroup per (group, head tile), then one per split
  // workgroup for its waves' descriptors (the host bounds the sum below 2^31)
  const int n_items = a.num_seqs * a.num_kv_heads * ((a.group * a.pos_count + 3) / 4);
  const dim3 grid((unsigned)((int64_t)n_append + n_items + a.bal_grid));
  EncodeArgs none{};
  none.dtype = TQ_BF16;
  const EncodeArgs &e = ea ? *ea : none;
  switch (e.dtype) {
    case TQ_BF16: hipLaunchKernelGGL(step_prep_kernel<TQ_BF16>, grid, dim3(256), 0, stream, e, a, n_append, n_items); break;
    case TQ_F16: hipLaunchKernelGGL(step_prep_kernel<TQ_F16>, grid, dim3(256), 0, stream, e, a, n_append, n_items); break;
    case TQ_F32: hipLaunchKernelGGL(step_prep_kernel<TQ_F32>, grid, dim3(256), 0, stream, e, a, n_append, n_items); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_seqs * a.q_len * a.num_q_heads;
  const unsigned row_blocks = (unsigned)((rows + 3) / 4);
  const int64_t groups = (int64_t)a.num_seqs * a.q_len * a.num_kv_heads;
  hipError_t e = hipSuccess;
  if (a.qk_tiles > 0) {  // matrix-core pass, its own query operands: a workgroup per (chunk, KV head)
    // rows = (position, head) pairs, at most 8 per workgroup: up to 4 query
    // rows take the one-tile-per-wave pass; 5 to 8, or several groups of
    // positions (all in one launch), the two-head-tile pass
    const int per = decode_positions_per_launch(a.group);
    const int64_t items = a.bal_grid;
    const int pgroups = (a.q_len + per - 1) / per;
    DecodeArgs la = a;
    la.pos0 = 0;
    la.pos_count = min(per, a.q_len);
    la.qk_tiles = (la.group * la.pos_count + 3) / 4;
    if (a.balanced == 2) {  // the stream plan (fused decode step, verify blocks): every position in one launch
      la.pos_count = a.q_len;
      la.qk_tiles = (la.group * la.pos_count + 3) / 4;
      if (la.qk_tiles > 8 || a.hot_parts > 0 || !a.qops) return hipErrorInvalidValue;
      hipLaunchKernelGGL((split_wave_kernel<1, true>), dim3((unsigned)items), dim3(256), 0, stream, la);
    } else if (pgroups == 1 && la.qk_tiles == 1) {
      // the exact window's chunks ride in the same launch (q_len 1)
      const int64_t hot_items = a.hot_parts > 0 ? (int64_t)a.num_seqs * a.num_kv_heads * a.hot_parts : 0;
      hipLaunchKernelGGL((split_wave_kernel<1, false>), dim3((unsigned)(items + hot_items)), dim3(256), 0, stream, la);
    } else if (la.qk_tiles == 2) {
      hipLaunchKernelGGL(split_mfma_kernel<2>, dim3((unsigned)(items * pgroups)), dim3(512), 0, stream, la);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL(query_prep_kernel, dim3((unsigned)groups, (unsigned)a.group), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (prefill_uses_mfma(a.q_len, a.group, a.cb.bits)) {
      e = launch_prefill(a, stream);
    } else {
      switch (group_capacity(a.group)) {
        case 1: e = launch_split<1>(a, stream); break;
        case 2: e = launch_split<2>(a, stream); break;
        case 4: e = launch_split<4>(a, stream); break;
        case 8: e = launch_split<8>(a, stream); break;
        case 16: e = launch_split<16>(a, stream); break;
        default: return hipErrorInvalidValue;
      }
    }
    if (e != hipSuccess) return e;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.hot_parts > 0 && a.qk_tiles != 1) {  // the exact window's records (unless folded above)
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_kv_heads * a.hot_parts));
    if (a.group < 1 || a.group > 16) return hipErrorInvalidValue;
    launch_hot(a, grid, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // four waves per row when there are more records than one batch
  if (a.balanced == 2)
    hipLaunchKernelGGL((merge_kernel<4, 32>), dim3((unsigned)rows), dim3(256), 0, stream, a, rows);
  else if (a.part_stride > kMergeBatch)
    hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)rows), dim3(256), 0, stream, a, rows);
  else
    hipLaunchKernelGGL(merge_kernel<1>, dim3(row_blocks), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

}  // namespace tq
