// Chunked-prefill attention over the compressed paged cache on the matrix
// cores (q_len > 1, causal): query t of a sequence of length L sees keys
// 0 .. L - q_len + t.
//
// Scores and values follow the bit-plane pages (SwiftLM README,
// "TurboQuantization: KV Cache Compression"; K keeps codes, QJL signs, norm
// and residual length, V codes and norm):
//   score(q, j) = scale * n_j * (<H q, c[idx_j]> + gamma_j <alpha S q, sigma_j>)
//   o' = sum_j p_j n^V_j c[vidx_j]  (rotated domain, one inverse WHT in merge)
//
// A workgroup of eight waves takes 128 query rows (128/G positions x G heads
// of one KV head) and a chunk of keys, 32 keys (two pages) per step.  Each
// step the waves dequantize the two K pages into f16 tiles in LDS (levels
// hi + lo, signs +-1) and the two V pages (levels hi + lo, transposed), then
// every wave computes, for its 16 rows (the tiles' LDS reads, about 40 KB
// per wave and step, bound the step rather than the matrix cores; two row
// tiles per wave would halve them but leave one wave per SIMD, which
// measured slower),
//   S^T = K Q^T  on v_mfma_f32_16x16x32_f16: codes in three passes
//        (K_hi Q_hi + K_hi Q_lo + K_lo Q_hi), signs in two (sigma S_hi +
//        sigma S_lo): hi + lo halves carry ~22 bits on both sides, which the
//        logits of large-norm keys need;
//   O^T += V^T W^T  with W = p n^V as the B operand straight from the score
//        registers (lane l holds one query row, so no transpose is needed):
//        three passes (V_hi W_hi + V_lo W_hi + V_hi W_lo).  A single f16 W
//        (2^-11 relative) left errors near 3e-3 of a row's largest output
//        where a dominant value's outlier channels cancel in the output.
// The running maximum is exact (W <= n^V fits f16); the partial record
// (m in log2 units, l, acc[128]) goes to the merge pass, which applies the
// inverse WHT.

#include "tq_common.hpp"

namespace tq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kPartStride = 132;  // m (log2 units), l, pad, pad, acc[128]
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeys = 32;         // keys per step (two pages)
constexpr float kTabScale = 16.0f;  // levels are tabulated x16: their lo halves stay normal f16

// One step's dequantized tiles, each stored in the order the matrix ops read
// it: entry [..][lane] is the 16-byte operand piece of lane 16 g + r, so a
// wave's operand read is one contiguous 1 KiB and no two lanes of it share
// a bank.  K tile (ct, kc): lane (g, r) holds coordinates 32 kc + 8 g .. +7
// of key 16 ct + r; V tile cv: lane (g, r) holds slots 8 g .. 8 g + 7 of
// coordinate 16 cv + r.
struct Tile {
  v8h kh[2][4][64];                // key levels x16, hi: [key tile][coordinate block][lane]
  v8h kl[2][4][64];                // lo
  v8h ks[2][4][64];                // QJL signs +-1
  v8h vh[8][64];                   // value levels x16, hi: [coordinate tile][lane]
  v8h vl[8][64];                   // lo
  float kn[2 * kKeys];             // n_k / 16 (entries past kKeys: copies no one reads)
  float kg[2 * kKeys];             // n_k gamma
  float vn[2 * kKeys];             // n_v
};

// Two steps in flight: the tiles of step i are read while those of step
// i + 1 are written, and the stored pages of step i + 1 are staged while
// those of step i are still being dequantized.
struct PrefillLds {
  Tile d[2];
  uint8_t rawk[2][2][kKPage];      // [buffer][page] as stored
  uint8_t rawv[2][2][kVPage];
};

// Four 3-bit codes (bytes of sel, 0..7) to four f16 values through byte
// tables: t0/t1 hold the low bytes of entries 0..3 / 4..7, u0/u1 the high
// bytes.  Returns f16 pairs (entries 0,1) and (2,3).
__device__ __forceinline__ uint2 lut4(uint32_t sel, uint32_t t0, uint32_t t1, uint32_t u0, uint32_t u1) {
  const uint32_t lo = __builtin_amdgcn_perm(t1, t0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(u1, u0, sel);
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

// Bits 0..3 of x to the lowest bit of bytes 0..3.
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 0xFu) * 0x00204081u) & 0x01010101u; }

// Code bytes of four coordinates (or tokens) from bit n, n+1, n+2, n+3 of
// the three plane words: idx = b0 + 2 b1 + 4 b2.
__device__ __forceinline__ uint32_t code_bytes(uint32_t p0, uint32_t p1, uint32_t p2, int n) {
  return spread4(p0 >> n) | (spread4(p1 >> n) << 1) | (spread4(p2 >> n) << 2);
}

// Two f16 +-1 per bit pair of s starting at bit n: sigma = 2 bit - 1.
__device__ __forceinline__ uint32_t sign_pair(uint32_t s, int n) {
  const uint32_t b0 = (s >> n) & 1u, b1 = (s >> (n + 1)) & 1u;
  return 0x3C003C00u | ((b0 ^ 1u) << 15) | ((b1 ^ 1u) << 31);
}

__device__ __forceinline__ float half_at(const uint8_t *p) {
  return (float)*reinterpret_cast<const _Float16 *>(p);
}

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowTiles = 1;                  // 16-row tiles per wave (each shares the tile reads)
constexpr int kRows = 16 * kRowTiles * kWaves;  // query rows per workgroup
static_assert(kRows == kPrefillRows, "the host plans prefill blocks of kPrefillRows rows");

// Dequantize a step's staged pages into T (all threads of the workgroup, one
// item of each kind per thread, no branch: the step's matrix ops and this
// vector work then share one basic block and interleave).  Keys: item (key,
// 8 coordinates), the key fastest along the lanes (the record bytes the
// lanes read then lie in distinct banks); values: item (coordinate, page,
// half of the page's tokens), tokens 4g..4g+3 of page pg going to slots 8g +
// 4pg .. +3 (the B operand order of the weights).  512 items of each kind.
static_assert(kThreads == 512, "one dequantization item of each kind per thread");
__device__ __forceinline__ void dequantize(Tile &T, const uint8_t (*rawk)[kKPage], const uint8_t (*rawv)[kVPage],
                                           int tid, const uint32_t (&th)[4], const uint32_t (&tl)[4]) {
  {
    const int it = tid;
    const int tok = it & 15, p16 = (it >> 4) & 15, pg = it >> 8;
    const uint8_t *pk = rawk[pg];
    // byte p16 of a token's 128-bit field: coordinates (rows) 8 p16 .. +7, in
    // byte p16 % 4 of that field's word of the record of chunk p16 / 4
    const int kb = k_record(p16 >> 2, tok) + (p16 & 3);
    const uint32_t w0 = pk[kb];
    const uint32_t w1 = pk[kb + 4];
    const uint32_t w2 = pk[kb + 8];
    const uint32_t ws = pk[kb + 4 * kKSignField];
    uint32_t hv[4], lv[4], sv[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t sel = code_bytes(w0, w1, w2, 4 * q);
      const uint2 hh = lut4(sel, th[0], th[1], th[2], th[3]);
      const uint2 ll = lut4(sel, tl[0], tl[1], tl[2], tl[3]);
      hv[2 * q] = hh.x;
      hv[2 * q + 1] = hh.y;
      lv[2 * q] = ll.x;
      lv[2 * q + 1] = ll.y;
      sv[2 * q] = sign_pair(ws, 4 * q);
      sv[2 * q + 1] = sign_pair(ws, 4 * q + 2);
    }
    // coordinates 8 p16 .. +7 = block p16 / 4, lane group p16 % 4
    const int kc = p16 >> 2, ln = 16 * (p16 & 3) + tok;
    *reinterpret_cast<uint4 *>(&T.kh[pg][kc][ln]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<uint4 *>(&T.kl[pg][kc][ln]) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
    *reinterpret_cast<uint4 *>(&T.ks[pg][kc][ln]) = make_uint4(sv[0], sv[1], sv[2], sv[3]);
  }
  {
    const int it = tid;
    const int r = it & 15, pg = (it >> 4) & 1, th8 = (it >> 5) & 1, cv = it >> 6, c = 16 * cv + r;
    const uint8_t *pv = rawv[pg];
    const uint32_t w0 = pv[kVPlane * 0 + 2 * c + th8];
    const uint32_t w1 = pv[kVPlane * 1 + 2 * c + th8];
    const uint32_t w2 = pv[kVPlane * 2 + 2 * c + th8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int g = 2 * th8 + q;
      const uint32_t sel = code_bytes(w0, w1, w2, 4 * q);
      // slots 8 g + 4 pg .. +3: half 4 pg of lane (g, r)'s piece
      _Float16 *vh = reinterpret_cast<_Float16 *>(&T.vh[cv][16 * g + r]) + 4 * pg;
      _Float16 *vl = reinterpret_cast<_Float16 *>(&T.vl[cv][16 * g + r]) + 4 * pg;
      *reinterpret_cast<uint2 *>(vh) = lut4(sel, th[0], th[1], th[2], th[3]);
      *reinterpret_cast<uint2 *>(vl) = lut4(sel, tl[0], tl[1], tl[2], tl[3]);
    }
  }
  {
    // threads 0..31 the 32 keys' norms; threads 32..63 copies to the unread
    // half (every thread past 63 repeats thread tid % 64's store)
    const int e = tid & (2 * kKeys - 1), pg = (e >> 4) & 1, tok = e & 15;
    const float nk = half_at(&rawk[pg][kKNorm + 2 * tok]);
    T.kn[e] = nk * (1.0f / kTabScale);
    T.kg[e] = nk * half_at(&rawk[pg][kKGamma + 2 * tok]);
    T.vn[e] = half_at(&rawv[pg][kVNorm + 2 * tok]);
  }
}

__global__ __launch_bounds__(kThreads, 1) void prefill_mfma_kernel(DecodeArgs a) {
  // G query heads per KV head (any of 1 .. 16): BQ whole positions per
  // workgroup, rows past BQ G unused
  const int G = a.group;
  const int BQ = kRows / G;  // query positions per workgroup
  const int qblocks = (a.q_len + BQ - 1) / BQ;
  const int b = blockIdx.x / qblocks, qb = blockIdx.x % qblocks;
  const int h = blockIdx.y, split = blockIdx.z;
  const int L = clamped_context(a, b);
  const int t0 = qb * BQ;
  const int t_last = min(t0 + BQ, a.q_len) - 1;
  const int s0 = seq_base(a, L) + split * a.split_tokens;
  const int s1 = min(min(s0 + a.split_tokens, L), L - a.q_len + t_last + 1);
  if (s0 >= s1) return;  // uniform: no key of the chunk is visible to the block
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  __shared__ __align__(16) PrefillLds S;

  // this lane's query rows (columns of S^T and O^T), one per row tile u
  bool row_ok[kRowTiles];
  int64_t R[kRowTiles];
  int lim[kRowTiles], low[kRowTiles];
#pragma unroll
  for (int u = 0; u < kRowTiles; ++u) {
    const int rw = 16 * (kRowTiles * wave + u) + l16;
    const int t = t0 + rw / G, hq = h * G + rw % G;
    row_ok[u] = t < a.q_len && rw < BQ * G;
    R[u] = ((int64_t)b * a.q_len + min(t, a.q_len - 1)) * a.num_q_heads + hq;
    lim[u] = L - a.q_len + t;  // last visible key of the row
    low[u] = window_low(a, lim[u] + 1);  // first one (with a window)
  }

  // B operands of S^T: chunk kc = 0..3 rotated query, 4..7 alpha S q, scaled
  // by softmax scale x log2(e), as f16 hi and lo
  v8h qh[kRowTiles][8], ql[kRowTiles][8];
  {
    const float cs = a.scale * kLog2e;
#pragma unroll
    for (int u = 0; u < kRowTiles; ++u) {
      const float *src = a.qprep + R[u] * 256;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const float4 x0 = *reinterpret_cast<const float4 *>(src + 32 * kc + 8 * g4);
        const float4 x1 = *reinterpret_cast<const float4 *>(src + 32 * kc + 8 * g4 + 4);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = row_ok[u] ? cs * xs[j] : 0.0f;
          const _Float16 hi = (_Float16)v;
          qh[u][kc][j] = hi;
          ql[u][kc][j] = (_Float16)(v - (float)hi);
        }
      }
    }
  }

  // byte tables of the levels x16 (hi and lo halves), uniform
  uint32_t th[4], tl[4];
  {
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float c = kTabScale * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.cb.c[k])));
      const _Float16 hi = (_Float16)c;
      const _Float16 lo = (_Float16)(c - (float)hi);
      hb[k] = __builtin_bit_cast(uint16_t, hi);
      lb[k] = __builtin_bit_cast(uint16_t, lo);
    }
    // th[0..1]: low bytes of hi entries 0..3 / 4..7, th[2..3]: high bytes
    th[0] = (hb[0] & 0xFF) | (hb[1] & 0xFF) << 8 | (hb[2] & 0xFF) << 16 | (hb[3] & 0xFF) << 24;
    th[1] = (hb[4] & 0xFF) | (hb[5] & 0xFF) << 8 | (hb[6] & 0xFF) << 16 | (hb[7] & 0xFF) << 24;
    th[2] = (hb[0] >> 8) | (hb[1] >> 8) << 8 | (hb[2] >> 8) << 16 | (hb[3] >> 8) << 24;
    th[3] = (hb[4] >> 8) | (hb[5] >> 8) << 8 | (hb[6] >> 8) << 16 | (hb[7] >> 8) << 24;
    tl[0] = (lb[0] & 0xFF) | (lb[1] & 0xFF) << 8 | (lb[2] & 0xFF) << 16 | (lb[3] & 0xFF) << 24;
    tl[1] = (lb[4] & 0xFF) | (lb[5] & 0xFF) << 8 | (lb[6] & 0xFF) << 16 | (lb[7] & 0xFF) << 24;
    tl[2] = (lb[0] >> 8) | (lb[1] >> 8) << 8 | (lb[2] >> 8) << 16 | (lb[3] >> 8) << 24;
    tl[3] = (lb[4] >> 8) | (lb[5] >> 8) << 8 | (lb[6] >> 8) << 16 | (lb[7] >> 8) << 24;
  }

  // arguments the lambdas below use, as locals (a captured argument struct
  // would be copied to scratch memory)
  const int32_t *const btab = a.block_tables + (int64_t)b * a.max_blocks;
  const uint8_t *const k_cache = a.k_cache, *const v_cache = a.v_cache;
  const int64_t hkv = a.num_kv_heads;
  // 16-byte piece of the step's pages loaded by this thread: K pieces
  // 0..135, V pieces 136..235
  auto load_raw = [&](int k0) {
    k0 = k0 < s1 ? k0 : s0;  // a step past the chunk re-reads the first one (never used)
    uint4 r = make_uint4(0u, 0u, 0u, 0u);
    if (tid < 2 * (kKPage / 16) + 2 * (kVPage / 16)) {
      const bool isk = tid < 2 * (kKPage / 16);
      const int q = isk ? tid : tid - 2 * (kKPage / 16);
      const int per = isk ? kKPage / 16 : kVPage / 16;
      const int pgi = q / per, off = 16 * (q % per);
      // a page past the chunk's end re-reads the step's first page (its keys
      // are masked)
      const int pg = (k0 + 16 * pgi < s1) ? (k0 >> 4) + pgi : (k0 >> 4);
      const int64_t blk = btab[page_entry(a, pg)];
      const uint8_t *base = isk ? k_cache + (blk * hkv + h) * kKPage : v_cache + (blk * hkv + h) * kVPage;
      r = *reinterpret_cast<const uint4 *>(base + off);
    }
    return r;
  };
  auto store_raw = [&](const uint4 &r, int buf) {
    if (tid < 2 * (kKPage / 16) + 2 * (kVPage / 16)) {
      const bool isk = tid < 2 * (kKPage / 16);
      const int q = isk ? tid : tid - 2 * (kKPage / 16);
      const int per = isk ? kKPage / 16 : kVPage / 16;
      uint8_t *dst = isk ? &S.rawk[buf][q / per][16 * (q % per)] : &S.rawv[buf][q / per][16 * (q % per)];
      *reinterpret_cast<uint4 *>(dst) = r;
    }
  };

  v4f acc[kRowTiles][8];
  float m_run[kRowTiles], l_part[kRowTiles];
#pragma unroll
  for (int u = 0; u < kRowTiles; ++u) {
    m_run[u] = -INFINITY;
    l_part[u] = 0.0f;
#pragma unroll
    for (int cv = 0; cv < 8; ++cv) acc[u][cv] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int nsteps = (s1 - s0 + kKeys - 1) / kKeys;
  uint4 raw = load_raw(s0);
  store_raw(raw, 0);
  lds_barrier();
  raw = load_raw(s0 + kKeys);
  dequantize(S.d[0], S.rawk[0], S.rawv[0], tid, th, tl);
  for (int st = 0; st < nsteps; ++st) {
    const int k0 = s0 + kKeys * st;
    const Tile &T = S.d[st & 1];
    store_raw(raw, (st + 1) & 1);
    // step st's tiles are complete, step st - 1's are consumed, and the
    // pages of step st + 1 are staged
    lds_barrier();
    raw = load_raw(k0 + 2 * kKeys);

    // ---- S^T = K Q^T for this wave's rows: lane l, register i of key tile
    // ct holds key 16 ct + 4 (l / 16) + i of row l % 16 of row tile u
    v4f cc[kRowTiles][2], csg[kRowTiles][2];
#pragma unroll
    for (int u = 0; u < kRowTiles; ++u)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) cc[u][ct] = csg[u][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const v8h ah = T.kh[ct][kc][lane];
        const v8h al = T.kl[ct][kc][lane];
        const v8h as = T.ks[ct][kc][lane];
#pragma unroll
        for (int u = 0; u < kRowTiles; ++u) {
          cc[u][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qh[u][kc], cc[u][ct], 0, 0, 0);
          cc[u][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ql[u][kc], cc[u][ct], 0, 0, 0);
          cc[u][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qh[u][kc], cc[u][ct], 0, 0, 0);
          csg[u][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as, qh[u][4 + kc], csg[u][ct], 0, 0, 0);
          csg[u][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as, ql[u][4 + kc], csg[u][ct], 0, 0, 0);
        }
      }
    }
    // tiles of step st + 1 (past the last step: unused), written while this
    // step's are read: independent of the score chains above, so their
    // vector work runs while the matrix cores do
    dequantize(S.d[(st + 1) & 1], S.rawk[(st + 1) & 1], S.rawv[(st + 1) & 1], tid, th, tl);
#pragma unroll
    for (int u = 0; u < kRowTiles; ++u) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        pin_result(cc[u][ct]);
        pin_result(csg[u][ct]);
      }
    }

    // ---- online softmax (log2 units), exact running maximum --------------
    float knv[2][4], kgv[2][4], vnv[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const float4 kn4 = *reinterpret_cast<const float4 *>(&T.kn[16 * ct + 4 * g4]);
      const float4 kg4 = *reinterpret_cast<const float4 *>(&T.kg[16 * ct + 4 * g4]);
      const float4 vn4 = *reinterpret_cast<const float4 *>(&T.vn[16 * ct + 4 * g4]);
      knv[ct][0] = kn4.x; knv[ct][1] = kn4.y; knv[ct][2] = kn4.z; knv[ct][3] = kn4.w;
      kgv[ct][0] = kg4.x; kgv[ct][1] = kg4.y; kgv[ct][2] = kg4.z; kgv[ct][3] = kg4.w;
      vnv[ct][0] = vn4.x; vnv[ct][1] = vn4.y; vnv[ct][2] = vn4.z; vnv[ct][3] = vn4.w;
    }
    v8h wb[kRowTiles], wbl[kRowTiles];
#pragma unroll
    for (int u = 0; u < kRowTiles; ++u) {
      float sc[2][4];
      bool vis[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * ct + 4 * g4 + i;
          vis[ct][i] = key < s1 && key <= lim[u] && key >= low[u];
          const float raw_s = fmaf(knv[ct][i], cc[u][ct][i], kgv[ct][i] * csg[u][ct][i]);
          sc[ct][i] = vis[ct][i] ? raw_s : -INFINITY;
          tmax = fmaxf(tmax, sc[ct][i]);
        }
      }
      tmax = fmaxf(tmax, xchg16(tmax, lane));
      tmax = fmaxf(tmax, xchg32(tmax, lane));
      const float m_new = fmaxf(m_run[u], tmax);
      // m_run = -inf: nothing accumulated yet (acc and l are zero)
      const float f = m_run[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[u] - m_new);
      m_run[u] = m_new;
      // f = 1 (exact) where the row's maximum did not move: no branch
      l_part[u] *= f;
#pragma unroll
      for (int cv = 0; cv < 8; ++cv) acc[u][cv] *= f;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = vis[ct][i] ? __builtin_amdgcn_exp2f(sc[ct][i] - m_new) : 0.0f;
          l_part[u] += p;
          // the norm of a masked key may hold any bits: its weight is selected to 0
          const float w = vis[ct][i] ? p * vnv[ct][i] : 0.0f;
          const _Float16 wh = (_Float16)w;
          wb[u][4 * ct + i] = wh;
          wbl[u][4 * ct + i] = (_Float16)(w - (float)wh);
        }
      }
    }

    // ---- O^T += V^T W^T: A = value levels [coordinate][slot] -------------
#pragma unroll
    for (int cv = 0; cv < 8; ++cv) {
      const v8h vh = T.vh[cv][lane];
      const v8h vl = T.vl[cv][lane];
#pragma unroll
      for (int u = 0; u < kRowTiles; ++u) {
        acc[u][cv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, wb[u], acc[u][cv], 0, 0, 0);
        acc[u][cv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, wb[u], acc[u][cv], 0, 0, 0);
        acc[u][cv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, wbl[u], acc[u][cv], 0, 0, 0);
      }
    }
  }

  // ---- partial records: the lanes of one row hold 4 key groups ----------
#pragma unroll
  for (int u = 0; u < kRowTiles; ++u) {
    float l_row = l_part[u] + xchg16(l_part[u], lane);
    l_row += xchg32(l_row, lane);
    if (row_ok[u]) {
      float *part = a.partials + (R[u] * a.part_stride + split) * kPartStride;
      if (g4 == 0) {
        part[0] = m_run[u];
        part[1] = l_row;
      }
#pragma unroll
      for (int cv = 0; cv < 8; ++cv) {
        const float4 o = make_float4(acc[u][cv][0], acc[u][cv][1], acc[u][cv][2], acc[u][cv][3]) * (1.0f / kTabScale);
        *reinterpret_cast<float4 *>(part + 4 + 16 * cv + 4 * g4) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const DecodeArgs &a, hipStream_t stream) {
  if (a.group < 1 || a.group > kMaxGroup) return hipErrorInvalidValue;
  const int bq = kRows / a.group;
  const int qblocks = (a.q_len + bq - 1) / bq;
  dim3 grid((unsigned)(a.num_seqs * qblocks), (unsigned)a.num_kv_heads, (unsigned)a.num_splits);
  hipLaunchKernelGGL(prefill_mfma_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
