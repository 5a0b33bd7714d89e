// Attention read directly from the compressed, paged cache (gfx950).
//
// Three launches on the caller's stream:
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

#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kPartStride = 132;  // m, l, pad, pad, acc[128]

// A context length above the planned maximum breaks the caller contract; it
// is cut to what the block table row and the split plan cover, so that no
// access leaves the block table or the partials.
__device__ __forceinline__ int clamped_context(const DecodeArgs &a, int b) {
  const int cap = min(a.max_blocks * kBlock, a.num_splits * a.split_tokens);
  return min(max(a.context_lens[b], 0), cap);
}

// ---- 1. query prep: a workgroup per 4 query rows ----------------------------
// Thread (i, half) keeps S[i][64*half .. +64) in registers (all 64 loads in
// flight at once), then forms the partial S q for each row; LDS adds the two
// halves.  The rotation runs on wave w for row w.
constexpr int kPrepRows = 4;

__global__ __launch_bounds__(256) void query_prep_kernel(DecodeArgs a, int64_t rows) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * kPrepRows;
  __shared__ float qs[kPrepRows][kHeadDim];
  __shared__ float part[2][kPrepRows][kHeadDim];
  const int64_t r = r0 + wave;
  float x0 = 0.0f, x1 = 0.0f;
  if (r < rows) {
    x0 = load_as_float(a.q, a.q_dtype, r * kHeadDim + lane);
    x1 = load_as_float(a.q, a.q_dtype, r * kHeadDim + 64 + lane);
  }
  qs[wave][lane] = x0;
  qs[wave][lane + 64] = x1;
  const int i = tid & 127, half = tid >> 7;
  float sk[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) sk[k] = a.St[(half * 64 + k) * kQjlDim + i];
  lds_barrier();
#pragma unroll
  for (int rr = 0; rr < kPrepRows; ++rr) {
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 64; ++k) acc = fmaf(sk[k], qs[rr][half * 64 + k], acc);
    part[half][rr][i] = acc;
  }
  lds_barrier();
  if (r >= rows) return;
  wave_fwht128(x0, x1, lane);
  float *out = a.qprep + r * 256;
  out[lane] = x0;
  out[lane + 64] = x1;
  out[128 + lane] = a.cb.qjl_scale * (part[0][wave][lane] + part[1][wave][lane]);
  out[128 + lane + 64] = a.cb.qjl_scale * (part[0][wave][lane + 64] + part[1][wave][lane + 64]);
}

// ---- 2. split pass (vector ALU) --------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void split_valu_kernel(DecodeArgs a) {
  const int bt = blockIdx.x;  // b * q_len + t
  const int h = blockIdx.y;
  const int split = blockIdx.z;
  const int b = bt / a.q_len, t = bt % a.q_len;
  const int L = clamped_context(a, b);
  const int vis = max(0, L - a.q_len + t + 1);
  const int s0 = split * a.split_tokens;
  const int s1 = min(s0 + a.split_tokens, vis);
  if (s0 >= s1) return;  // uniform: this chunk holds no visible key
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // main loop: qp[G][128] | sq[G][128] | pn[4][G][64]; after it: red[4][G][128]
  __shared__ float smem[G * 512];
  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ float lut[8];
  float *qp = smem;
  float *sq = smem + G * 128;
  float *pn = smem + G * 256;

  const int64_t row0 = (int64_t)bt * a.num_q_heads + (int64_t)h * G;
  for (int idx = tid; idx < G * 256; idx += 256) {
    const int g = idx >> 8, c = idx & 255;
    const float v = a.qprep[(row0 + g) * 256 + c];
    if (c < 128) qp[g * 128 + c] = v; else sq[g * 128 + c - 128] = v;
  }
  if (tid < 8) {
    // read the levels into registers first: a select over kernel-argument
    // fields can be folded into a lane-indexed memory load
    float cv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cv[j] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.c[j])));
    float c = cv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) c = (tid == j) ? cv[j] : c;
    lut[tid] = c;
  }
  lds_barrier();

  const int32_t *btab = a.block_tables + (int64_t)b * a.max_blocks;
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
    const bool valid = (c < nchunks) && (j < s1);
    float score[G];
    float nv = 0.0f;
    if (valid) {
      const int64_t page = (int64_t)btab[j >> 4] * a.num_kv_heads + h;
      const int o = j & 15;
      const uint8_t *kp = a.k_cache + page * kKPage;
      const uint4 P0 = *reinterpret_cast<const uint4 *>(kp + 16 * o);
      const uint4 P1 = *reinterpret_cast<const uint4 *>(kp + kKPlane + 16 * o);
      const uint4 P2 = *reinterpret_cast<const uint4 *>(kp + 2 * kKPlane + 16 * o);
      const uint4 Q = *reinterpret_cast<const uint4 *>(kp + kKSigns + 16 * o);
      const float nk = (float)*reinterpret_cast<const _Float16 *>(kp + kKNorm + 2 * o);
      const float gm = (float)*reinterpret_cast<const _Float16 *>(kp + kKGamma + 2 * o);
      nv = (float)*reinterpret_cast<const _Float16 *>(a.v_cache + page * kVPage + kVNorm + 2 * o);
      const uint32_t w0[4] = {P0.x, P0.y, P0.z, P0.w};
      const uint32_t w1[4] = {P1.x, P1.y, P1.z, P1.w};
      const uint32_t w2[4] = {P2.x, P2.y, P2.z, P2.w};
      const uint32_t wq[4] = {Q.x, Q.y, Q.z, Q.w};
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
          const int idx = ((w0[w] >> bb) & 1) | (((w1[w] >> bb) & 1) << 1) | (((w2[w] >> bb) & 1) << 2);
          const float cv = lut[idx];
          const float sg = ((wq[w] >> bb) & 1) ? 1.0f : -1.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            dk[g] = fmaf(qp[g * 128 + i], cv, dk[g]);
            ds[g] = fmaf(sq[g * 128 + i], sg, ds[g]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) score[g] = a.scale * nk * fmaf(gm, ds[g], dk[g]);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) score[g] = -INFINITY;
    }
    // online softmax, wave-wide per head
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(m[g], wave_max(score[g]));
      const float p = (mn == -INFINITY) ? 0.0f : __expf(score[g] - mn);
      const float corr = (mn == -INFINITY) ? 1.0f : __expf(m[g] - mn);
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
        const uint8_t *vp = a.v_cache + ((int64_t)btab[tok0 >> 4] * a.num_kv_heads + h) * kVPage;
        const uint32_t a0 = *reinterpret_cast<const uint16_t *>(vp + 2 * lane);
        const uint32_t a1 = *reinterpret_cast<const uint16_t *>(vp + kKPlane + 2 * lane);
        const uint32_t a2 = *reinterpret_cast<const uint16_t *>(vp + 2 * kKPlane + 2 * lane);
        const uint32_t b0 = *reinterpret_cast<const uint16_t *>(vp + 128 + 2 * lane);
        const uint32_t b1 = *reinterpret_cast<const uint16_t *>(vp + kKPlane + 128 + 2 * lane);
        const uint32_t b2 = *reinterpret_cast<const uint16_t *>(vp + 2 * kKPlane + 128 + 2 * lane);
#pragma unroll 4
        for (int tt = 0; tt < 16; ++tt) {
          const int ia = ((a0 >> tt) & 1) | (((a1 >> tt) & 1) << 1) | (((a2 >> tt) & 1) << 2);
          const int ib = ((b0 >> tt) & 1) | (((b1 >> tt) & 1) << 1) | (((b2 >> tt) & 1) << 2);
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
  for (int idx = tid; idx < G * 128; idx += 256) {
    const int g = idx >> 7, d = idx & 127;
    float M = red_m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][g]);
    float Ls = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (red_m[w][g] == -INFINITY) ? 0.0f : __expf(red_m[w][g] - M);
      Ls = fmaf(f, red_l[w][g], Ls);
      A = fmaf(f, red[(w * G + g) * 128 + d], A);
    }
    float *part = a.partials + ((row0 + g) * a.num_splits + split) * kPartStride;
    if (d == 0) {
      part[0] = M;
      part[1] = Ls;
    }
    part[4 + d] = A;
  }
}

// ---- 3. merge: one wave per output row --------------------------------------
// Lanes read the chunk maxima and sums in parallel; the weighted sum of the
// chunk accumulators issues its loads eight chunks at a time.
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int64_t rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  __shared__ float fw[4][64];
  if (r >= rows) return;
  const int64_t per_seq = (int64_t)a.q_len * a.num_q_heads;
  const int b = (int)(r / per_seq);
  const int t = (int)((r / a.num_q_heads) % a.q_len);
  const int L = clamped_context(a, b);
  const int vis = max(0, L - a.q_len + t + 1);
  const int ns = (vis + a.split_tokens - 1) / a.split_tokens;
  const float *part = a.partials + r * a.num_splits * kPartStride;
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, part[s * kPartStride]);
  M = wave_max(M);
  float Ls = 0.0f, A0 = 0.0f, A1 = 0.0f;
  for (int base = 0; base < ns; base += 64) {
    const int s = base + lane;
    float f = 0.0f;
    if (s < ns) {
      const float m = part[s * kPartStride];
      f = (m == -INFINITY) ? 0.0f : __expf(m - M);
      Ls = fmaf(f, part[s * kPartStride + 1], Ls);
    }
    fw[wave][lane] = f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int cnt = min(64, ns - base);
    int u = 0;
    for (; u + 8 <= cnt; u += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float *p = part + (int64_t)(base + u + e) * kPartStride + 4;
        v0[e] = p[lane];
        v1[e] = p[64 + lane];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f2 = fw[wave][u + e];
        A0 = fmaf(f2, v0[e], A0);
        A1 = fmaf(f2, v1[e], A1);
      }
    }
    for (; u < cnt; ++u) {
      const float *p = part + (int64_t)(base + u) * kPartStride + 4;
      const float f2 = fw[wave][u];
      A0 = fmaf(f2, p[lane], A0);
      A1 = fmaf(f2, p[64 + lane], A1);
    }
    __builtin_amdgcn_wave_barrier();
  }
  Ls = wave_sum(Ls);
  float o0 = 0.0f, o1 = 0.0f;
  if (Ls > 0.0f) {
    const float inv = 1.0f / Ls;
    o0 = A0 * inv;
    o1 = A1 * inv;
  }
  wave_fwht128(o0, o1, lane);
  store_from_float(a.out, a.out_dtype, r * kHeadDim + lane, o0);
  store_from_float(a.out, a.out_dtype, r * kHeadDim + 64 + lane, o1);
}

template <int G>
hipError_t launch_split(const DecodeArgs &a, hipStream_t stream) {
  dim3 grid((unsigned)(a.num_seqs * a.q_len), (unsigned)a.num_kv_heads, (unsigned)a.num_splits);
  hipLaunchKernelGGL(split_valu_kernel<G>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_seqs * a.q_len * a.num_q_heads;
  const unsigned row_blocks = (unsigned)((rows + 3) / 4);
  hipLaunchKernelGGL(query_prep_kernel, dim3((unsigned)((rows + kPrepRows - 1) / kPrepRows)),
                     dim3(256), 0, stream, a, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.group) {
    case 1: e = launch_split<1>(a, stream); break;
    case 2: e = launch_split<2>(a, stream); break;
    case 4: e = launch_split<4>(a, stream); break;
    case 8: e = launch_split<8>(a, stream); break;
    case 16: e = launch_split<16>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(row_blocks), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

}  // namespace tq
