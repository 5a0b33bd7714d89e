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

#include "tq_mfma.hpp"

namespace tq {
namespace {

constexpr int kPartStride = 132;  // m (log2 units), l, pad, pad, acc[128]
constexpr float kLog2e = 1.4426950408889634f;

// LSE combine of the chunk partials of output row r by one wave, o' = acc'/l,
// one inverse FWHT, store.  Lane l owns coordinates l and l + 64.  The chunk
// accumulators are loaded 32 chunks at a time, the first batch issued before
// the maxima are reduced, so a typical row costs one round trip to memory;
// lane e computes the weight of chunk base + e and readlane broadcasts it.
__device__ void merge_row(const DecodeArgs &a, int64_t r, int lane) {
  const int64_t per_seq = (int64_t)a.q_len * a.num_q_heads;
  const int b = (int)(r / per_seq);
  const int t = (int)((r / a.num_q_heads) % a.q_len);
  const int L = clamped_context(a, b);
  const int vis = max(0, L - a.q_len + t + 1);
  const int ns = (vis + a.split_tokens - 1) / a.split_tokens;
  const float *part = a.partials + r * a.num_splits * kPartStride;
  constexpr int kBatch = 32;
  float v0[kBatch], v1[kBatch];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const float *p = part + (int64_t)max(min(base + e, ns - 1), 0) * kPartStride;
      v0[e] = p[4 + lane];
      v1[e] = p[68 + lane];
    }
  };
  if (ns > 0) load_batch(0);
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, part[(int64_t)s * kPartStride]);
  M = wave_max(M);
  float Ls = 0.0f, A0 = 0.0f, A1 = 0.0f;
  for (int base = 0; base < ns; base += kBatch) {
    if (base > 0) load_batch(base);
    const int se = base + (lane & (kBatch - 1));
    float f = 0.0f;
    if (se < ns && lane < kBatch) {
      const float m = part[(int64_t)se * kPartStride];
      f = (m == -INFINITY) ? 0.0f : exp2f(m - M);
      Ls = fmaf(f, part[(int64_t)se * kPartStride + 1], Ls);
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const float fe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), e));  // 0 past ns
      A0 = fmaf(fe, v0[e], A0);
      A1 = fmaf(fe, v1[e], A1);
    }
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

// ---- 1. query prep: a workgroup per query row --------------------------------
// Grid (sequence x position x KV head, head of the group).  Thread (i, half)
// forms half of (S q)_i from S[i][64*half .. +64) held in registers; wave 0
// rotates q.  For the matrix-core pass the workgroup also writes its head's
// rows of the score contraction's A operands (see split_mfma_kernel): rows
// (head, digit r).  With 2^E bounding |x| over the head, Y = rint(x 2^(19-E))
// is written in balanced base 32, Y = d0 2^15 + d1 2^10 + d2 2^5 + d3 with
// every |d_r| <= 16, stored as the fp6 e2m3 code of d_r/8 (exact), and row r
// carries it with scale 2^(E-4-5r+3): x to 2^-20 of the head's largest
// magnitude.  Logits of keys with large norms need these 19 bits; 16
// (base-16 digits) leave errors near 1e-3 in peaked rows.
__device__ __forceinline__ int bound_exponent(float M) {  // M < 2^E for finite M > 0
  const int ex = (int)((__float_as_uint(M) >> 23) & 0xFFu);
  return ex == 0 ? -126 : ex - 126;
}

__global__ __launch_bounds__(256) void query_prep_kernel(DecodeArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int64_t grp = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t row = grp * G + g;
  __shared__ float qs[kHeadDim];
  __shared__ float part[2][kQjlDim];
  __shared__ float qp[256];
  __shared__ float hmax[2];
  __shared__ float cpart[2][8];
  if (tid < kHeadDim) qs[tid] = load_as_float(a.q, a.q_dtype, row * kHeadDim + tid);
  const int i = tid & 127, half = tid >> 7;
  float sk[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) sk[k] = a.St[(half * 64 + k) * kQjlDim + i];
  lds_barrier();
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 64; ++k) acc = fmaf(sk[k], qs[half * 64 + k], acc);
  part[half][i] = acc;
  if (wave == 0) {
    float x0 = qs[lane], x1 = qs[lane + 64];
    wave_fwht128(x0, x1, lane);
    qp[lane] = x0;
    qp[lane + 64] = x1;
    const float mq = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    if (lane == 0) hmax[0] = mq;
  }
  lds_barrier();
  if (tid < kQjlDim) qp[128 + tid] = a.cb.qjl_scale * (part[0][tid] + part[1][tid]);
  lds_barrier();
  a.qprep[row * 256 + tid] = qp[tid];
  if (a.qa == nullptr) return;

  if (wave == 1) {
    const float ms = wave_max(fmaxf(fabsf(qp[128 + lane]), fabsf(qp[192 + lane])));
    if (lane == 0) hmax[1] = ms;
  }
  lds_barrier();
  float beta[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) beta[p] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.beta[p])));
  // per plane: 2^E bounds |x| (E >= -100 keeps every scale encodable); no
  // digits at all when the plane is zero
  int Ep[5];
  bool nz[5];
#pragma unroll
  for (int p = 0; p < 5; ++p) {
    const float M = p < 4 ? fabsf(beta[p]) * hmax[0] : hmax[1];
    nz[p] = M > 0.0f;
    Ep[p] = max(bound_exponent(M), -100);
  }
  const int NT = a.qk_tiles;
  const int nwords = NT * 5 * 64 * 8;
  const int nt = g >> 2, gp = g & 3;
  uint32_t *qa = a.qa + grp * (int64_t)(NT * (5 * 64 * 9 + 32));
  __shared__ __align__(16) uint8_t codes[5][4][128];  // [plane][digit][K slot] fp6 codes
  __shared__ float spart[4][8];                       // per wave: start-value partial sums
  // 1. digits of every (plane, K slot): the four digits of one value go to
  // four A rows.  The digit of a K slot is scaled by the factor that goes
  // with the b_split operands; the start values (per digit r, the weighted
  // sum of the unscaled A values, see b_split) are summed on the way, for the
  // code planes (p < 4) and the sign plane.
  float sc4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sq4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int e = tid; e < 5 * 128; e += 256) {
    const int p = e >> 7, kap = e & 127;
    const bool pz = p == 0 ? nz[0] : p == 1 ? nz[1] : p == 2 ? nz[2] : p == 3 ? nz[3] : nz[4];
    const int E = p == 0 ? Ep[0] : p == 1 ? Ep[1] : p == 2 ? Ep[2] : p == 3 ? Ep[3] : Ep[4];
    const float bp = p == 0 ? beta[0] : p == 1 ? beta[1] : p == 2 ? beta[2] : beta[3];
    const float x = p < 4 ? -bp * qp[b_coord(kap)] : -qp[128 + b_coord(kap)];
    // Y = rint(x 2^(19-E)) = d0 2^15 + d1 2^10 + d2 2^5 + d3, |d_r| <= 16
    const float y = pz ? rintf(ldexpf(x, 19 - E)) : 0.0f;
    const float d0 = rintf(y * 0x1p-15f);
    float rem = y - d0 * 32768.0f;
    const float d1 = rintf(rem * 0x1p-10f);
    rem -= d1 * 1024.0f;
    const float d2 = rintf(rem * 0.03125f);
    const float d3 = rem - d2 * 32.0f;
    const float f = b_split_factor(kap), wgt = b_split_weight(kap);
    codes[p][0][kap] = (uint8_t)fp6_code(d0 * f);
    codes[p][1][kap] = (uint8_t)fp6_code(d1 * f);
    codes[p][2][kap] = (uint8_t)fp6_code(d2 * f);
    codes[p][3][kap] = (uint8_t)fp6_code(d3 * f);
    const float v0 = wgt * ldexpf(d0, E - 4), v1 = wgt * ldexpf(d1, E - 9);
    const float v2 = wgt * ldexpf(d2, E - 14), v3 = wgt * ldexpf(d3, E - 19);
    if (p < 4) {
      sc4[0] += v0; sc4[1] += v1; sc4[2] += v2; sc4[3] += v3;
    } else {
      sq4[0] += v0; sq4[1] += v1; sq4[2] += v2; sq4[3] += v3;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc4[r] = wave_sum(sc4[r]);
    sq4[r] = wave_sum(sq4[r]);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      spart[wave][r] = sc4[r];
      spart[wave][4 + r] = sq4[r];
    }
  }
  lds_barrier();
  // 2. this head's rows: lanes 16*ga + 4*gp + r of tile nt, 32 fp6 codes (K
  // slot 32 ga + s at code s) packed into six words, and their E8M0 scales
  if (tid < 5 * 16) {
    const int li = tid & 15, p = tid >> 4;
    const int ga = li >> 2, r = li & 3, ln = 16 * ga + 4 * gp + r;
    const uint4 c0 = *reinterpret_cast<const uint4 *>(&codes[p][r][32 * ga]);
    const uint4 c1 = *reinterpret_cast<const uint4 *>(&codes[p][r][32 * ga + 16]);
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    // four 6-bit codes per byte-word to 24 bits, eight of those to six words
    uint32_t q24[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t v = cw[k];
      q24[k] = (v & 0x3Fu) | ((v >> 2) & 0xFC0u) | ((v >> 4) & 0x3F000u) | ((v >> 6) & 0xFC0000u);
    }
    uint32_t w[6];
#pragma unroll
    for (int k = 0; k < 2; ++k) {  // 4 x 24 bits = 3 words
      w[3 * k + 0] = q24[4 * k] | (q24[4 * k + 1] << 24);
      w[3 * k + 1] = (q24[4 * k + 1] >> 8) | (q24[4 * k + 2] << 16);
      w[3 * k + 2] = (q24[4 * k + 2] >> 16) | (q24[4 * k + 3] << 8);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(qa + ((nt * 5 + p) * 64 + ln) * 8);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], 0u, 0u);
    const bool pz = p == 0 ? nz[0] : p == 1 ? nz[1] : p == 2 ? nz[2] : p == 3 ? nz[3] : nz[4];
    const int E = p == 0 ? Ep[0] : p == 1 ? Ep[1] : p == 2 ? Ep[2] : p == 3 ? Ep[3] : Ep[4];
    qa[nwords + (nt * 5 + p) * 64 + ln] = (uint32_t)(pz ? min(E - 4 - 5 * r + kFp6Exp + kE8M0One, 254) : kE8M0One);
  }
  if (tid < 8)
    qa[nwords + NT * 5 * 64 + (nt * 4 + gp) * 8 + tid] =
        __float_as_uint((spart[0][tid] + spart[1][tid]) + (spart[2][tid] + spart[3][tid]));
  // rows of absent heads (groups of one or two heads) stay zero
  if (g == 0 && G < 4) {
    for (int i = tid; i < (4 - G) * 8; i += 256) qa[nwords + NT * 5 * 64 + G * 8 + i] = 0u;
    for (int widx = tid; widx < 5 * 64 * 8; widx += 256) {
      const int ln = (widx >> 3) & 63;
      if (((ln & 15) >> 2) >= G) qa[widx] = 0u;
    }
    for (int sidx = tid; sidx < 5 * 64; sidx += 256) {
      const int ln = sidx & 63;
      if (((ln & 15) >> 2) >= G) qa[nwords + sidx] = (uint32_t)kE8M0One;
    }
  }
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
      const float f = (red_m[w][g] == -INFINITY) ? 0.0f : exp2f(red_m[w][g] - M);
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

// ---- 2'. split pass on the matrix cores (single-query decode, G <= 8) -----
// Both contractions run on the scaled f8f6f4 MFMA, with the stored bits as
// the fp4 operand (B = 1 - 2 bit, one and_or per 8 values) and the float side
// split into four digits in four A rows: the query side in balanced base 32
// as fp6 codes (see query_prep_kernel; fp6 x fp4 runs at twice the fp8 x fp4
// rate), the weights in base 16 as fp8.  With the bit-plane form
// of the levels, c[idx] = -(beta0 B0 + beta1 B1 + beta2 B2 + beta3 Bx) where
// Bx = B0 B1 B2 is the plane of b0^b1^b2:
//   <q', c[idx]> = sum_p <-beta_p q', B_p>        (4 MFMAs per page)
//   gamma <s, sigma> = gamma <-s, B_sign>          (1 MFMA per page)
//   o' = -sum_p beta_p sum_j w_j B_p,j  with w_j = p_j n_v,j  (4 planes)
// A workgroup (4 waves) walks its chunk in tiles of 128 tokens (8 pages).
// Wave w scores pages 2w, 2w+1 of a tile (MFMA K-block w of the value
// contraction), keeps the block maximum m_w (integer, log2 units) and writes
// the digits of w_j / 2^E_w to LDS; 2^(E_w + m_w - m) enters as the E8M0
// scale of K-block w, so no cross-wave agreement on exponents is needed.
// The value contraction is split by coordinates: wave w owns N-tiles 2w and
// 2w+1 (32 coordinates) for all four planes.  The running maximum m is
// shared by all waves and moves only when a tile exceeds it by 2^64.
struct MfmaTile {
  uint8_t wq[4][4][128];   // [head][digit][K] fp8 digits of w
  uint32_t vs[4][400];     // [page pair][plane * 128 + coord], padded
  float mi[4][4];          // [head][K-block] block maxima (log2 units)
  int ex[4][4];            // [head][K-block] digit exponents
};

struct MfmaLoads {
  uint4 kr[2];                 // K page records: plane lane/16, token lane%16
  uint32_t nk[2], gm[2], nv[2];
  uint4 vp[2];                 // value planes of the wave's page pair (lanes < 48)
};

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
__device__ __forceinline__ float half_bits(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ float sel4(const float (&v)[4], int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// 4x4 transpose of (16-lane row, register): row g register j -> row j register g.
__device__ __forceinline__ void transpose_rows(uint32_t &r0, uint32_t &r1, uint32_t &r2, uint32_t &r3) {
  const auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

// Block ids of a wave's pages, one per lane: lane j holds page j & 1 of the
// wave's page pair in tile base + j/2 (32 tiles per register), so a tile's
// page addresses come from readlane with no memory round trip.  A page past
// the visible range re-reads its tile's first page (always visible; its
// tokens are masked), and a tile past the chunk the chunk's first page.
__device__ __forceinline__ int wave_page_ids(const int32_t *btab, int s0, int s1, int base, int wave, int lane) {
  const int tile0 = s0 + 128 * (base + (lane >> 1));
  const int tok = tile0 + 16 * (2 * wave + (lane & 1));
  const int pg = tile0 >= s1 ? (s0 >> 4) : ((tok < s1 ? tok : tile0) >> 4);
  return btab[pg];
}

// The two pages (block ids b0, b1, uniform) of the wave's page pair: K
// records (plane lane/16, token lane%16), the scalars, and the value planes.
__device__ __forceinline__ void mfma_load_tile(MfmaLoads &R, const uint8_t *k_cache, const uint8_t *v_cache,
                                               int64_t hkv, int h, int b0, int b1, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int64_t blk = kk == 0 ? b0 : b1;
    const uint8_t *kp = k_cache + (blk * hkv + h) * kKPage;
    const uint8_t *vp = v_cache + (blk * hkv + h) * kVPage;
    R.kr[kk] = *reinterpret_cast<const uint4 *>(kp + 16 * lane);
    R.nk[kk] = *reinterpret_cast<const uint16_t *>(kp + kKNorm + 2 * (lane & 15));
    R.gm[kk] = *reinterpret_cast<const uint16_t *>(kp + kKGamma + 2 * (lane & 15));
    R.nv[kk] = *reinterpret_cast<const uint16_t *>(vp + kVNorm + 2 * (lane & 15));
    // value planes of the wave's own page pair: lane < 48 takes 16 bytes
    if (lane < 48) R.vp[kk] = *reinterpret_cast<const uint4 *>(vp + kKPlane * (lane >> 4) + 16 * (lane & 15));
  }
}

// A workgroup serves one chunk of one KV head and up to four of its query
// heads (one operand tile); eight heads per KV head take two workgroups whose
// dispatch ids differ by 8, so that they run on the same XCD at the same time
// and the second reads the pages from L2.  Each barrier interval holds two
// independent chains for the scheduler to interleave: the value contraction
// of tile i-1 and the scores and weight digits of tile i.
struct SplitItem {
  int b, h, hh, split;
  bool ok;
};
__device__ __forceinline__ SplitItem split_item(const DecodeArgs &a, int halves) {
  const int lin = blockIdx.x;
  SplitItem it;
  int item;
  if (halves == 2) {
    item = 8 * (lin >> 4) + (lin & 7);
    it.hh = (lin >> 3) & 1;
  } else {
    item = lin;
    it.hh = 0;
  }
  const int per_seq = a.num_kv_heads * a.num_splits;
  it.ok = item < a.num_seqs * per_seq;
  item = it.ok ? item : 0;
  it.b = item / per_seq;
  it.h = (item / a.num_splits) % a.num_kv_heads;
  it.split = item % a.num_splits;
  return it;
}

__global__ __launch_bounds__(256, 2) void split_mfma_kernel(DecodeArgs a) {
  const int halves = a.qk_tiles;
  const SplitItem item = split_item(a, halves);
  if (!item.ok) return;  // uniform: padding of the interleaved grid
  const int b = item.b, h = item.h, hh = item.hh, split = item.split;
  const int L = clamped_context(a, b);
  const int s0 = split * a.split_tokens;
  const int s1 = min(s0 + a.split_tokens, L);
  if (s0 >= s1) return;  // uniform
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t16 = lane & 15, grow = lane >> 4;
  const int64_t grp = (int64_t)b * a.num_kv_heads + h;
  const int G = a.group;

  __shared__ __align__(16) MfmaTile buf[2];
  __shared__ float lred[4][4];

  // query-side operands of the score contraction: tile hh of the group
  v8i Aq[5];
  int scq[5];
  v4f cinit, qinit;  // accumulator start values (see b_split)
  {
    const uint32_t *qa = a.qa + grp * (int64_t)(halves * (5 * 64 * 9 + 32));
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const uint4 *src = reinterpret_cast<const uint4 *>(qa + ((hh * 5 + p) * 64 + lane) * 8);
      const uint4 u0 = src[0];
      const uint2 u1 = *reinterpret_cast<const uint2 *>(src + 1);
      Aq[p] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, 0, 0};
      scq[p] = (int)qa[halves * 5 * 64 * 8 + (hh * 5 + p) * 64 + lane];
    }
    const float *ci = reinterpret_cast<const float *>(qa + halves * 5 * 64 * 9) + (hh * 4 + grow) * 8;
    cinit = v4f{ci[0], ci[1], ci[2], ci[3]};
    qinit = v4f{ci[4], ci[5], ci[6], ci[7]};
  }
  float beta[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) beta[p] = uniform(a.cb.beta[p]);
  const float cs = a.scale * kLog2e;
  const int32_t *const btab = a.block_tables + (int64_t)b * a.max_blocks;
  const uint8_t *const k_cache = a.k_cache, *const v_cache = a.v_cache;
  const int64_t hkv = a.num_kv_heads;
  const int ntiles = (s1 - s0 + 127) >> 7;
  // block ids of this wave's pages, 32 tiles per register (the next 32 are
  // fetched a block ahead)
  int ids_cur = wave_page_ids(btab, s0, s1, 0, wave, lane);
  int ids_nxt = ntiles > 32 ? wave_page_ids(btab, s0, s1, 32, wave, lane) : 0;
  int ids_base = 0;
  auto load_tile = [&](MfmaLoads &R, int k) {
    if (k >= ids_base + 32) {  // uniform
      ids_cur = ids_nxt;
      ids_base += 32;
      if (ids_base + 32 < ntiles) ids_nxt = wave_page_ids(btab, s0, s1, ids_base + 32, wave, lane);
    }
    const int j = 2 * (k - ids_base);
    mfma_load_tile(R, k_cache, v_cache, hkv, h, __builtin_amdgcn_readlane(ids_cur, j),
                   __builtin_amdgcn_readlane(ids_cur, j + 1), lane);
  };

  float mref[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // shared running maximum per head
  float lsum = 0.0f;
  v4f acc[4][2];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[p][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const int gA = t16 >> 2, rA = lane & 3, kb = grow;  // A-operand row and scale block of this lane

  // Scores of pages 2*wave, 2*wave+1 of the tile at tok0 (lane: head grow,
  // token t16), their block maximum and the weight digits, into Bf; returns
  // the lane's probability sum and block maximum through ps, mi.  The matrix
  // ops write all 64 lanes whatever the exec mask, so they must never sit
  // under a lane-dependent branch: every lane computes its score, and keys
  // past the visible range are masked afterwards with a select.
  auto scores = [&](const MfmaLoads &R, int tok0, MfmaTile &Bf, float &ps, float &mi) {
    float sc[2];
    bool valid[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t r0 = R.kr[kk].x, r1 = R.kr[kk].y, r2 = R.kr[kk].z, r3 = R.kr[kk].w;
      transpose_rows(r0, r1, r2, r3);  // now plane p's word grow in r_p, signs in r3
      const v8i B0 = b_split(r0), B1 = b_split(r1), B2 = b_split(r2), Bx = b_split(r0 ^ r1 ^ r2),
                Bs = b_split(r3);
      const float nk = half_bits(R.nk[kk] & 0xFFFFu), gm = half_bits(R.gm[kk] & 0xFFFFu);
      valid[kk] = tok0 + 16 * (2 * wave + kk) + t16 < s1;
      v4f c = mfma_f6f4(Aq[0], B0, cinit, scq[0]);
      c = mfma_f6f4(Aq[1], B1, c, scq[1]);
      c = mfma_f6f4(Aq[2], B2, c, scq[2]);
      c = mfma_f6f4(Aq[3], Bx, c, scq[3]);
      const v4f q = mfma_f6f4(Aq[4], Bs, qinit, scq[4]);
      const float code = (c[0] + c[1]) + (c[2] + c[3]);
      const float qj = (q[0] + q[1]) + (q[2] + q[3]);
      float raw = cs * nk * fmaf(gm, qj, code);
      // pin the score (and the matrix ops feeding it) to the unconditional
      // path: otherwise they may be sunk into the branch of the select below
      asm volatile("" : "+v"(raw));
      sc[kk] = valid[kk] ? raw : -INFINITY;
    }
    mi = ceilf(row_max16(fmaxf(sc[0], sc[1])));
    float w[2];
    ps = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const float p = sc[kk] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[kk] - mi);
      ps += p;
      // the norm of a slot past the visible range may hold any bits
      w[kk] = (valid[kk] && p > 0.0f) ? p * half_bits(R.nv[kk] & 0xFFFFu) : 0.0f;
    }
    const float wm = row_max16(fmaxf(w[0], w[1]));
    const int E = wm > 0.0f ? bound_exponent(wm) : 0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t X = (uint32_t)fminf(rintf(ldexpf(w[kk], 16 - E)), 65535.0f);
      uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32((float)(X >> 12), (float)((X >> 8) & 15u), 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32((float)((X >> 4) & 15u), (float)(X & 15u), pk, true);
      const int kap = b_kappa(32 * wave + 16 * kk + t16);
#pragma unroll
      for (int r = 0; r < 4; ++r) Bf.wq[grow][r][kap] = (uint8_t)(pk >> (8 * r));
    }
    if (t16 == 0) {
      Bf.mi[grow][wave] = mi;
      Bf.ex[grow][wave] = E;
    }
    // value planes of this wave's page pair: interleave the 16-bit words
    if (lane < 48) {
      const uint4 &va = R.vp[0], &vb = R.vp[1];
      const uint32_t sel_lo = 0x05040100u, sel_hi = 0x07060302u;
      uint4 o0, o1;
      o0.x = __builtin_amdgcn_perm(vb.x, va.x, sel_lo);
      o0.y = __builtin_amdgcn_perm(vb.x, va.x, sel_hi);
      o0.z = __builtin_amdgcn_perm(vb.y, va.y, sel_lo);
      o0.w = __builtin_amdgcn_perm(vb.y, va.y, sel_hi);
      o1.x = __builtin_amdgcn_perm(vb.z, va.z, sel_lo);
      o1.y = __builtin_amdgcn_perm(vb.z, va.z, sel_hi);
      o1.z = __builtin_amdgcn_perm(vb.w, va.w, sel_lo);
      o1.w = __builtin_amdgcn_perm(vb.w, va.w, sel_hi);
      uint4 *dst = reinterpret_cast<uint4 *>(&Bf.vs[wave][128 * (lane >> 4) + 8 * (lane & 15)]);
      dst[0] = o0;
      dst[1] = o1;
    }
  };

  // Value contraction of a tile whose digits are in Bf (after the barrier),
  // with the lane's probability sum ps and block maximum mi of that tile.
  auto values = [&](const MfmaTile &Bf, float ps, float mi) {
    // shared running maximum: moves only when a tile exceeds it by 2^64
    bool moved = false;
    float fct[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 m4 = *reinterpret_cast<const float4 *>(&Bf.mi[g][0]);
      const float Mt = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
      fct[g] = 1.0f;
      if (Mt > mref[g] + 64.0f) {
        fct[g] = __builtin_amdgcn_exp2f(mref[g] - Mt);
        mref[g] = Mt;
        moved = true;
      }
    }
    if (moved) {
      const float f = sel4(fct, grow);
      lsum *= f;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[p][j] *= f;
    }
    if (ps > 0.0f) lsum += ps * __builtin_amdgcn_exp2f(mi - sel4(mref, grow));
    // weight operand: row (head gA, digit rA), K-block scale from wave kb
    const uint4 u0 = *reinterpret_cast<const uint4 *>(&Bf.wq[gA][rA][16 * grow]);
    const uint4 u1 = *reinterpret_cast<const uint4 *>(&Bf.wq[gA][rA][64 + 16 * grow]);
    const v8i Aw = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
    const float mb = Bf.mi[gA][kb];
    int sw = kE8M0One;
    if (mb != -INFINITY) {
      const float d = fmaxf(mb - sel4(mref, gA), -300.0f);
      sw = min(max(Bf.ex[gA][kb] - 4 - 4 * rA + (int)d + kE8M0One, 0), 254);
    }
    // this wave's coordinates 32*wave .. +31
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 16 * (2 * wave + j) + t16;
      const uint32_t p0 = Bf.vs[grow][col], p1 = Bf.vs[grow][128 + col], p2 = Bf.vs[grow][256 + col];
      const v8i V0 = b_pm1(p0), V1 = b_pm1(p1), V2 = b_pm1(p2), Vx = b_pm1(p0 ^ p1 ^ p2);
      acc[0][j] = mfma_f8f4(Aw, V0, acc[0][j], sw);
      acc[1][j] = mfma_f8f4(Aw, V1, acc[1][j], sw);
      acc[2][j] = mfma_f8f4(Aw, V2, acc[2][j], sw);
      acc[3][j] = mfma_f8f4(Aw, Vx, acc[3][j], sw);
    }
  };

  MfmaLoads RA, RB;
  float psA = 0.0f, miA = -INFINITY, psB = 0.0f, miB = -INFINITY;
  load_tile(RA, 0);
  if (ntiles > 1) load_tile(RB, 1);
  scores(RA, s0, buf[0], psA, miA);
  // tile i (odd: RB, buf[1]; even: RA, buf[0]) with the values of tile i-1
  for (int i = 1; i < ntiles; i += 2) {
    if (i + 1 < ntiles) load_tile(RA, i + 1);
    lds_barrier();
    values(buf[0], psA, miA);
    scores(RB, s0 + 128 * i, buf[1], psB, miB);
    if (i + 1 >= ntiles) break;
    if (i + 2 < ntiles) load_tile(RB, i + 2);
    lds_barrier();
    values(buf[1], psB, miB);
    scores(RA, s0 + 128 * (i + 1), buf[0], psA, miA);
  }
  lds_barrier();
  if (ntiles & 1)
    values(buf[0], psA, miA);
  else
    values(buf[1], psB, miB);

  // row sums over the 16 lanes of a head, then over the waves
  {
    const float ls = row_sum16(lsum);
    if (t16 == 0) lred[wave][grow] = ls;
  }
  lds_barrier();
  const int g = 4 * hh + grow;
  if (g < G) {
    float *part = a.partials + ((grp * G + g) * a.num_splits + split) * kPartStride;
    if (wave == 0 && t16 == 0) {
      part[0] = sel4(mref, grow);
      part[1] = (lred[0][grow] + lred[1][grow]) + (lred[2][grow] + lred[3][grow]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float o = 0.0f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const v4f &c = acc[p][j];
        o = fmaf(-beta[p], (c[0] + c[1]) + (c[2] + c[3]), o);
      }
      part[4 + 16 * (2 * wave + j) + t16] = o;
    }
  }
}

// ---- 3. merge: one wave per output row --------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int64_t rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  merge_row(a, r, lane);
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
  const int64_t groups = (int64_t)a.num_seqs * a.q_len * a.num_kv_heads;
  hipLaunchKernelGGL(query_prep_kernel, dim3((unsigned)groups, (unsigned)a.group), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.qa != nullptr) {  // matrix-core pass: one workgroup per (chunk, KV head, head tile)
    if (a.qk_tiles != 1 && a.qk_tiles != 2) return hipErrorInvalidValue;
    const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads * a.num_splits;
    const int64_t wgs = a.qk_tiles == 1 ? items : 2 * ((items + 7) / 8) * 8;
    hipLaunchKernelGGL(split_mfma_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
  } else if (prefill_uses_mfma(a.q_len, a.group)) {
    e = launch_prefill(a, stream);
    if (e != hipSuccess) return e;
  } else {
    switch (a.group) {
      case 1: e = launch_split<1>(a, stream); break;
      case 2: e = launch_split<2>(a, stream); break;
      case 4: e = launch_split<4>(a, stream); break;
      case 8: e = launch_split<8>(a, stream); break;
      case 16: e = launch_split<16>(a, stream); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(row_blocks), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

}  // namespace tq
