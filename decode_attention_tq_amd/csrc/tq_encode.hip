// Fused TurboQuant encoder for gfx950.
//
// One workgroup (4 waves) takes 16 consecutive tokens of one KV head and, for
// each token, both its key and its value (SwiftLM README, "TurboQuantization:
// KV Cache Compression", K-cache steps 1-5 and the V-cache paragraph):
//   wave pass   : load x (coalesced, 2 coordinates per lane), norm by a wave
//                 reduction, normalise, in-register FWHT, fp32 threshold
//                 search, code bit-planes by ballot, residual in the rotated
//                 domain, its length, and the residual rotated back (one more
//                 FWHT) into LDS;
//   block pass  : QJL projection z = S r of the 16 key residuals (S^T streamed
//                 from L2, residuals broadcast from LDS), sign bits by ballot;
//   value planes: the coordinate-major V bit-planes gather one bit per token,
//                 so the 16 tokens' bits are merged per destination page; a
//                 page filled completely by this workgroup is stored, a
//                 partly filled one is updated with 32-bit atomic and/or.

#include "tq_common.hpp"

namespace tq {
namespace {

constexpr int kEncTokens = 16;

__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kEncTokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ float rk[kEncTokens][kHeadDim];       // key residual, original domain
  __shared__ uint8_t vcode[kEncTokens][kHeadDim];  // value codes
  __shared__ float lut[8];
  __shared__ int blk[kEncTokens], off[kEncTokens], valid[kEncTokens], leader[kEncTokens];

  if (tid < kEncTokens) {
    const int64_t t = t0 + tid;
    const int64_t s = (t < a.num_tokens) ? a.slots[t] : -1;
    valid[tid] = s >= 0;
    blk[tid] = s >= 0 ? (int)(s / kBlock) : -1;
    off[tid] = s >= 0 ? (int)(s % kBlock) : 0;
  }
  if (tid >= 32 && tid < 40) {
    const int k = tid - 32;
    float c = a.cb.c[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) c = (k == j) ? a.cb.c[j] : c;
    lut[k] = c;
  }
  __syncthreads();
  if (tid < kEncTokens) {
    int lead = valid[tid];
    for (int u = 0; u < tid; ++u)
      if (valid[u] && blk[u] == blk[tid]) lead = 0;
    leader[tid] = lead;
  }

  // ---- per-vector pass: one wave per (token, K or V) ----------------------
  for (int j = wave; j < kEncTokens; j += 4) {
    if (!valid[j]) continue;  // uniform across the wave
    const int64_t t = t0 + j;
    const int64_t base = t * a.tok_stride + (int64_t)h * a.head_stride;
    const int64_t page = (int64_t)blk[j] * a.num_kv_heads + h;
    uint8_t *kp = a.k_cache + page * kKPage;
    uint8_t *vp = a.v_cache + page * kVPage;
    const int o = off[j];

    // key: steps 1-4
    float x0 = load_as_float(a.k, a.dtype, base + lane);
    float x1 = load_as_float(a.k, a.dtype, base + lane + 64);
    const float nk = sqrtf(wave_sum(x0 * x0 + x1 * x1));
    const float invk = nk > 0.0f ? 1.0f / nk : 0.0f;
    float y0 = x0 * invk, y1 = x1 * invk;
    wave_fwht128(y0, y1, lane);
    const int i0 = cell_index(y0, a.cb), i1 = cell_index(y1, a.cb);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const uint64_t lo = __ballot((i0 >> p) & 1);
      const uint64_t hi = __ballot((i1 >> p) & 1);
      if (lane == 0)
        *reinterpret_cast<uint4 *>(kp + kKPlane * p + 16 * o) =
            make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
    }
    float e0 = y0 - lut[i0], e1 = y1 - lut[i1];
    const float gam = sqrtf(wave_sum(e0 * e0 + e1 * e1));
    wave_fwht128(e0, e1, lane);  // residual back in the original domain (H is its own inverse)
    rk[j][lane] = e0;
    rk[j][lane + 64] = e1;

    // value: steps 1-3
    x0 = load_as_float(a.v, a.dtype, base + lane);
    x1 = load_as_float(a.v, a.dtype, base + lane + 64);
    const float nv = sqrtf(wave_sum(x0 * x0 + x1 * x1));
    const float invv = nv > 0.0f ? 1.0f / nv : 0.0f;
    y0 = x0 * invv;
    y1 = x1 * invv;
    wave_fwht128(y0, y1, lane);
    vcode[j][lane] = (uint8_t)cell_index(y0, a.cb);
    vcode[j][lane + 64] = (uint8_t)cell_index(y1, a.cb);

    if (lane == 0) {
      *reinterpret_cast<_Float16 *>(kp + kKNorm + 2 * o) = to_half_sat(nk);
      *reinterpret_cast<_Float16 *>(kp + kKGamma + 2 * o) = to_half_sat(gam);
      *reinterpret_cast<_Float16 *>(vp + kVNorm + 2 * o) = to_half_sat(nv);
      if (a.norms_out) {
        float *no = a.norms_out + (t * a.num_kv_heads + h) * 3;
        no[0] = nk;
        no[1] = gam;
        no[2] = nv;
      }
    }
  }
  __syncthreads();

  // ---- QJL projection of the key residuals: z_i = sum_k S[i][k] r_k -------
  {
    const int i = tid & 127;
    const int grp = tid >> 7;  // tokens grp*8 .. grp*8+7; one group per wave
    float z[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) z[u] = 0.0f;
    for (int k = 0; k < kHeadDim; ++k) {
      const float s = a.St[k * kQjlDim + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) z[u] = fmaf(s, rk[grp * 8 + u][k], z[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = grp * 8 + u;
      const uint64_t bits = __ballot(z[u] >= 0.0f);
      if (valid[j] && lane == 0) {
        uint8_t *kp = a.k_cache + ((int64_t)blk[j] * a.num_kv_heads + h) * kKPage;
        const int ibase = (tid & 64);  // first row held by this wave
        *reinterpret_cast<uint2 *>(kp + kKSigns + 16 * off[j] + ibase / 8) =
            make_uint2((uint32_t)bits, (uint32_t)(bits >> 32));
      }
    }
  }

  // ---- value bit-planes: one 16-bit word per (plane, coordinate) ----------
  for (int w = tid; w < 3 * kHeadDim; w += 256) {
    const int p = w / kHeadDim, i = w % kHeadDim;
    for (int j = 0; j < kEncTokens; ++j) {
      if (!leader[j]) continue;
      uint32_t mask = 0, bits = 0;
      for (int u = j; u < kEncTokens; ++u) {
        if (valid[u] && blk[u] == blk[j]) {
          mask |= 1u << off[u];
          bits |= (uint32_t)((vcode[u][i] >> p) & 1) << off[u];
        }
      }
      uint8_t *vp = a.v_cache + ((int64_t)blk[j] * a.num_kv_heads + h) * kVPage;
      uint8_t *word = vp + kKPlane * p + 2 * i;
      if (mask == 0xFFFFu) {
        *reinterpret_cast<uint16_t *>(word) = (uint16_t)bits;
      } else {
        const uintptr_t addr = reinterpret_cast<uintptr_t>(word);
        uint32_t *w32 = reinterpret_cast<uint32_t *>(addr & ~uintptr_t(3));
        const int sh = (addr & 2) ? 16 : 0;
        const uint32_t set = bits << sh, clr = (mask & ~bits) << sh;
        if (clr) atomicAnd(w32, ~clr);
        if (set) atomicOr(w32, set);
      }
    }
  }
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream) {
  const int64_t groups = (a.num_tokens + kEncTokens - 1) / kEncTokens;
  dim3 grid((unsigned)groups, (unsigned)a.num_kv_heads, 1);
  hipLaunchKernelGGL(encode_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
