// C-ABI host layer of libtq: argument checking, the Lloyd-Max codebook and
// QJL matrix (double precision on the host), workspace planning and kernel
// dispatch.  Every check happens before any HIP call, so rejected calls touch
// nothing on the device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tq_status hip_fail(hipError_t e, const char *what) {
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- Lloyd-Max for N(0,1), symmetric half ---------------------------------
// The levels of a symmetric density come in +- pairs and (for an even count)
// the middle threshold is 0, so only the positive cells are iterated:
// cells (0, t_1], (t_1, t_2], ..., (t_{n-1}, inf) with levels c_1 < ... < c_n,
// t_k = (c_k + c_{k+1}) / 2, c_k = E[X | cell k] = (phi(a) - phi(b)) / (Q(a) - Q(b))
// (lilting.ch article, "Lloyd-Maxコードブックとは": levels fitted to the known
// N(0, 1/d) density by the Lloyd-Max iteration, once, before inference).

double std_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

double std_q(double x) {  // P(X > x), x >= 0
  if (std::isinf(x)) return 0.0;
  return 0.5 * std::erfc(x / std::sqrt(2.0));
}

void lloyd_max_positive_half(int half, std::vector<double> &c) {
  c.resize(half);
  for (int k = 0; k < half; ++k) c[k] = (k + 0.5) * (2.0 / half);  // any increasing start
  std::vector<double> edge(half + 1);
  for (int it = 0; it < 100000; ++it) {
    edge[0] = 0.0;
    for (int k = 1; k < half; ++k) edge[k] = 0.5 * (c[k - 1] + c[k]);
    edge[half] = INFINITY;
    double moved = 0.0;
    for (int k = 0; k < half; ++k) {
      const double a = edge[k], b = edge[k + 1];
      const double nc = (std_pdf(a) - std_pdf(b)) / (std_q(a) - std_q(b));
      moved = std::fmax(moved, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (moved < 1e-15) break;
  }
}

bool codebook_supported(int head_dim, int bits, int qjl_dim) {
  return head_dim == tq::kHeadDim && bits >= 2 && bits <= 4 && qjl_dim == tq::kQjlDim;
}
// Bit width of an initialised codebook (3 for a struct that is not one: the
// size queries accept any pointer).
int cb_bits(const tq_codebook *cb) { return cb && cb->magic == tq::kMagic ? cb->bits : 3; }

tq_status check_cb(const tq_codebook *cb) {
  if (!cb) return fail(TQ_ERR_INVALID_ARGUMENT, "codebook is NULL");
  if (cb->magic != tq::kMagic) return fail(TQ_ERR_NOT_INITIALIZED, "codebook not initialised by tq_codebook_init");
  if (!cb->d_tables) return fail(TQ_ERR_NOT_INITIALIZED, "codebook has no device tables");
  return TQ_OK;
}

tq::Codebook device_codebook(const tq_codebook *cb) {
  tq::Codebook d;
  std::memset(&d, 0, sizeof d);
  const int n = 1 << cb->bits;
  for (int i = 0; i < n; ++i) d.c[i] = cb->centroids[i];
  for (int i = 0; i + 1 < n; ++i) d.t[i] = cb->thresholds[i];
  d.bits = cb->bits;
  d.qjl_scale = cb->qjl_scale;
  if (cb->bits != 3) return d;  // the bit-plane form serves the 3-bit matrix-core passes
  // c4 = -b0 - b1 + b2 + b3, c5 = b0 - b1 + b2 - b3, c6 = -b0 + b1 + b2 - b3,
  // c7 = b0 + b1 + b2 + b3 (signs of B_p at the codes 4..7), solved in double.
  const double c4 = cb->centroids[4], c5 = cb->centroids[5], c6 = cb->centroids[6],
               c7 = cb->centroids[7];
  d.beta[0] = (float)((-c4 + c5 - c6 + c7) / 4.0);
  d.beta[1] = (float)((-c4 - c5 + c6 + c7) / 4.0);
  d.beta[2] = (float)((c4 + c5 + c6 + c7) / 4.0);
  d.beta[3] = (float)((c4 - c5 - c6 + c7) / 4.0);
  return d;
}

bool dtype_ok(int d) { return d == TQ_F32 || d == TQ_F16 || d == TQ_BF16; }

// ---- split-K planning ------------------------------------------------------
// The plan depends only on the call's sizes (no device query), so the
// workspace size and the launch always agree.
//
// Matrix-core decode pass (q_len = 1 or a short verify block, up to 8 query
// heads per KV head): the balanced plan.  Every (sequence, KV head) group is
// cut into ranges of `per` 128-token tiles, one workgroup each; per is chosen
// on the device from the actual context lengths as the smallest multiple of
// 4 in [4, 64] whose ranges fit in the count that fills the 256 compute units
// once (one 8-wave workgroup per unit for 5 to 8 query rows, two 4-wave ones
// for up to 4), so a ragged batch keeps the workgroups about equally busy.
// Each workgroup pays a fixed start-up (block ids, query operands, the first
// tiles in flight), so longer ranges are preferred once the units are full;
// a range holds at most 64 tiles (its block ids are kept in LDS).  The grid
// covers the ranges at per = 64 for every sequence at max_ctx; workgroups
// past the last range exit.  Records per row: k = ceil(T / per) <= T / 4,
// and below 64 tiles Hkv k fits the filling count.
// Other passes (vector pass, prefill): chunks of split_tokens (multiples of
// 256) per (sequence or query block, KV head), aiming at about 1024
// workgroups.
struct SplitPlan {
  int split_tokens, num_splits;  // num_splits: partial records per row (compressed part)
  int balanced, grid, target, per, min_tiles;
};
constexpr int kBalMinTiles = 4;  // and per is a multiple of 4 (one tile per wave and step)
constexpr int kBalMaxTiles = tq::kMaxMfmaSplitTokens / 128;

SplitPlan plan_splits(int num_seqs, int q_len, int num_kv_heads, int group, int max_ctx, int requested,
                      int bits) {
  SplitPlan p{};
  if (tq::decode_uses_mfma(q_len, group, bits)) {
    const int mrows = group * std::min(q_len, tq::decode_positions_per_launch(group));
    const long slots = mrows > 4 ? 256 : 512;
    const long tmax = (std::max(max_ctx, 0) + 127) / 128;
    const long groups = (long)num_seqs * num_kv_heads;
    p.balanced = 1;
    p.min_tiles = kBalMinTiles;
    p.target = (int)slots;
    long recs;
    if (requested > 0) {
      p.per = requested / 128;
      const long k = (tmax + p.per - 1) / p.per;
      p.grid = (int)std::max(1L, groups * k);
      recs = k;
    } else {
      p.per = 0;
      const long k64 = (tmax + kBalMaxTiles - 1) / kBalMaxTiles;
      p.grid = (int)std::max(slots, groups * k64);
      recs = std::max(std::min((tmax + kBalMinTiles - 1) / kBalMinTiles, slots / num_kv_heads), k64);
    }
    p.num_splits = (int)std::max(1L, std::min(recs, tmax));
    p.split_tokens = 128;
    return p;
  }
  int st;
  if (requested > 0) {
    st = requested;
  } else {
    long per_seq = q_len;
    if (tq::prefill_uses_mfma(q_len, group, bits)) {
      const int bq = tq::prefill_block_queries(group);
      per_seq = ((long)q_len + bq - 1) / bq;
    }
    const long rows = (long)num_seqs * per_seq * num_kv_heads;
    long want = (1024 + rows - 1) / rows;
    if (want < 1) want = 1;
    long per = (max_ctx + want - 1) / want;
    per = ((per + 255) / 256) * 256;
    if (per < 256) per = 256;
    st = (int)per;
  }
  p.split_tokens = st;
  p.num_splits = max_ctx > 0 ? (int)(((int64_t)max_ctx + st - 1) / st) : 1;
  return p;
}

constexpr size_t kPartStride = 132;  // floats per partial record: m, l, pad, pad, acc[128]

}  // namespace

namespace tq {
size_t decode_qprep_floats(int64_t rows) { return (size_t)rows * 256; }
size_t decode_partial_floats(int64_t rows, int parts) {
  return (size_t)rows * (size_t)parts * kPartStride;
}
int decode_hot_parts(int hot_max) { return hot_max > 0 ? (hot_max + kHotChunk - 1) / kHotChunk : 0; }
// A workgroup of the matrix-core decode pass takes at most 8 query rows
// (positions x heads) of a KV head, two 16-row operand tiles; more positions
// run as one launch per group of 8 / group of them, each reading the cache
// once.  Up to 4 such launches beat one prefill pass (measured at 32,768 and
// 131,072 cached tokens); beyond, the prefill pass takes the block.
bool decode_uses_mfma(int q_len, int group, int bits) {
  if (bits != 3 || q_len < 1 || group < 1 || group > 8) return false;
  const int per = 8 / group;
  return (q_len + per - 1) / per <= 4;
}
int decode_positions_per_launch(int group) { return 8 / group; }
// Longer query blocks of 3-bit caches take the matrix-core prefill pass.
bool prefill_uses_mfma(int q_len, int group, int bits) {
  return bits == 3 && q_len > 1 && !decode_uses_mfma(q_len, group, bits) && group >= 1 && group <= kMaxGroup;
}
int prefill_block_queries(int group) { return kPrefillRows / group; }
int decode_qk_tiles(int rows) { return (rows + 3) / 4; }
}  // namespace tq

extern "C" {

const char *tq_last_error(void) { return g_last_error.c_str(); }

tq_status tq_codebook_compute(int head_dim, int bits, float *centroids, float *thresholds) {
  if (!centroids || !thresholds) return fail(TQ_ERR_INVALID_ARGUMENT, "null output array");
  if (bits < 1 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be in [1, 4], got %d", bits);
  if (head_dim < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "head_dim must be positive");
  const int levels = 1 << bits, half = levels / 2;
  std::vector<double> pos;
  lloyd_max_positive_half(half, pos);
  const double s = std::sqrt((double)head_dim);
  for (int k = 0; k < half; ++k) {
    centroids[half + k] = (float)(pos[k] / s);
    centroids[half - 1 - k] = (float)(-pos[k] / s);
  }
  thresholds[half - 1] = 0.0f;
  for (int k = 1; k < half; ++k) {
    const double t = 0.5 * (pos[k - 1] + pos[k]);
    thresholds[half - 1 + k] = (float)(t / s);
    thresholds[half - 1 - k] = (float)(-t / s);
  }
  return TQ_OK;
}

tq_status tq_qjl_matrix(uint64_t seed, int rows, int cols, float *out) {
  if (!out) return fail(TQ_ERR_INVALID_ARGUMENT, "null output");
  if (rows < 1 || cols < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "rows and cols must be positive");
  uint64_t state = seed;
  auto next = [&state]() -> uint64_t {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  };
  const long n = (long)rows * cols;
  for (long k = 0; k < n; k += 2) {
    const double u1 = ((double)(next() >> 11) + 0.5) * 0x1.0p-53;
    const double u2 = ((double)(next() >> 11) + 0.5) * 0x1.0p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double th = 2.0 * M_PI * u2;
    out[k] = (float)(r * std::cos(th));
    if (k + 1 < n) out[k + 1] = (float)(r * std::sin(th));
  }
  return TQ_OK;
}

size_t tq_codebook_device_bytes(int head_dim, int qjl_dim) {
  if (head_dim < 1 || qjl_dim < 1) return 0;
  const size_t n = (size_t)head_dim * (size_t)qjl_dim;
  return 2 * n * sizeof(float) + 2 * n * sizeof(uint16_t);
}

tq_status tq_codebook_init(tq_codebook *cb, int head_dim, int bits, uint64_t qjl_seed,
                           const float *qjl_host, void *d_tables, void *stream) {
  if (!cb) return fail(TQ_ERR_INVALID_ARGUMENT, "codebook is NULL");
  if (!d_tables) return fail(TQ_ERR_INVALID_ARGUMENT, "d_tables is NULL");
  if ((uintptr_t)d_tables % 16 != 0) return fail(TQ_ERR_INVALID_ARGUMENT, "d_tables must be 16-byte aligned");
  if (!codebook_supported(head_dim, bits, tq::kQjlDim))
    return fail(TQ_ERR_UNSUPPORTED, "only head_dim=128 with bits 2, 3 or 4 are supported (got %d, %d)", head_dim,
                bits);
  tq_codebook c;
  std::memset(&c, 0, sizeof c);
  c.head_dim = head_dim;
  c.bits = bits;
  c.qjl_dim = tq::kQjlDim;
  c.block_size = tq::kBlock;
  c.qjl_seed = qjl_host ? 0 : qjl_seed;
  tq_status st = tq_codebook_compute(head_dim, bits, c.centroids, c.thresholds);
  if (st != TQ_OK) return st;
  c.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / tq::kQjlDim);
  const int m = tq::kQjlDim, d = head_dim;
  std::vector<float> host(2 * (size_t)m * d);
  if (qjl_host) {
    std::memcpy(host.data(), qjl_host, sizeof(float) * m * d);
  } else {
    st = tq_qjl_matrix(qjl_seed, m, d, host.data());
    if (st != TQ_OK) return st;
  }
  for (int i = 0; i < m; ++i)
    for (int k = 0; k < d; ++k) host[(size_t)m * d + (size_t)k * m + i] = host[(size_t)i * d + k];
  // S H (the projection applied to a residual that is still in the rotated
  // domain: S r = S H^T e = (S H) e, H symmetric), in double, then split into
  // a half "hi" part and a half "lo" part of the remainder for the matrix
  // cores: hi + lo carries ~22 significant bits.  The halves are stored in
  // the order the encoder's matrix operands take them, so that every lane
  // reads whole 16-byte pieces: for wave w, row tile u, K step k, part
  // (hi, lo) and lane l, eight halves j = 0..7 of row 16 (2w + u) + l % 16 at
  // column 16 j + 4 k + l / 16.
  std::vector<double> sh((size_t)m * d);
  const double inv_sqrt_d = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < m; ++i) {
    for (int k = 0; k < d; ++k) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) {
        const double hjk = (__builtin_popcount((unsigned)(j & k)) & 1) ? -inv_sqrt_d : inv_sqrt_d;
        acc += (double)host[(size_t)i * d + j] * hjk;
      }
      sh[(size_t)i * d + k] = acc;
    }
  }
  std::vector<uint16_t> halves(2 * (size_t)m * d);
  size_t o = 0;
  for (int w = 0; w < 4; ++w)
    for (int u = 0; u < 2; ++u)
      for (int k = 0; k < 4; ++k)
        for (int part = 0; part < 2; ++part)
          for (int l = 0; l < 64; ++l)
            for (int j = 0; j < 8; ++j) {
              const double v = sh[(size_t)(16 * (2 * w + u) + (l & 15)) * d + 16 * j + 4 * k + (l >> 4)];
              const _Float16 hi = (_Float16)v;
              const _Float16 h = part == 0 ? hi : (_Float16)(v - (double)hi);
              std::memcpy(&halves[o++], &h, 2);
            }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(d_tables, host.data(), host.size() * sizeof(float),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(tables)");
  e = hipMemcpyAsync((char *)d_tables + host.size() * sizeof(float), halves.data(),
                     halves.size() * sizeof(uint16_t), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(tables)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  // the no-allocation decode call's scratch address on this device, resolved
  // here at set-up so that the call itself never loads or allocates anything
  e = tq::noalloc_scratch(nullptr);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  c.d_tables = d_tables;
  c.magic = tq::kMagic;
  *cb = c;
  return TQ_OK;
}

size_t tq_k_page_bytes(const tq_codebook *cb) { return cb ? (size_t)tq::k_page_bytes(cb_bits(cb)) : 0; }
size_t tq_v_page_bytes(const tq_codebook *cb) { return cb ? (size_t)tq::v_page_bytes(cb_bits(cb)) : 0; }

}  // extern "C"

namespace {
// Checks of an encode call and its kernel arguments (shared by tq_encode_kv
// and the fused decode step); *launch is false for an empty call.
tq_status encode_args(const tq_codebook *cb, const void *k, const void *v, tq_dtype in_dtype, int64_t num_tokens,
                      int num_kv_heads, int64_t tok_stride, int64_t head_stride, const int64_t *slot_mapping,
                      uint8_t *k_cache, uint8_t *v_cache, float *norms_out, tq::EncodeArgs &a, bool *launch) {
  *launch = false;
  tq_status st = check_cb(cb);
  if (st != TQ_OK) return st;
  if (num_tokens < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (num_kv_heads < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "num_kv_heads must be >= 1");
  if (num_kv_heads > 65535) return fail(TQ_ERR_UNSUPPORTED, "num_kv_heads > 65535");
  if (!dtype_ok(in_dtype)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown in_dtype %d", (int)in_dtype);
  if (num_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(TQ_ERR_INVALID_ARGUMENT, "null device pointer");
  if (tok_stride < 0 || head_stride < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "negative stride");
  if (num_tokens > 1 && tok_stride < tq::kHeadDim && head_stride < tq::kHeadDim)
    return fail(TQ_ERR_INVALID_ARGUMENT, "strides overlap the 128 contiguous coordinates");
  if ((num_tokens + 15) / 16 > 0x7fffffffLL) return fail(TQ_ERR_UNSUPPORTED, "num_tokens too large");
  {
    // inputs are read 16 bytes per lane: 8 coordinates (4 for fp32) at a time
    const int64_t vec = in_dtype == TQ_F32 ? 4 : 8;
    if (tok_stride % vec != 0 || head_stride % vec != 0 ||
        (reinterpret_cast<uintptr_t>(k) & 15) != 0 || (reinterpret_cast<uintptr_t>(v) & 15) != 0)
      return fail(TQ_ERR_UNSUPPORTED,
                  "k and v must be 16-byte aligned with strides that are multiples of %d elements",
                  (int)vec);
  }
  a.k = k;
  a.v = v;
  a.dtype = in_dtype;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.tok_stride = tok_stride;
  a.head_stride = head_stride;
  a.slots = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.norms_out = norms_out;
  a.S = (const float *)cb->d_tables;
  a.St = (const float *)cb->d_tables + (size_t)tq::kQjlDim * tq::kHeadDim;
  a.SHop = (const uint16_t *)(a.St + (size_t)tq::kQjlDim * tq::kHeadDim);
  a.cb = device_codebook(cb);
  *launch = true;
  return TQ_OK;
}
}  // namespace

extern "C" {

tq_status tq_encode_kv(const tq_codebook *cb, const void *k, const void *v, tq_dtype in_dtype,
                       int64_t num_tokens, int num_kv_heads, int64_t tok_stride,
                       int64_t head_stride, const int64_t *slot_mapping, uint8_t *k_cache,
                       uint8_t *v_cache, float *norms_out, void *stream) {
  tq::EncodeArgs a;
  bool launch;
  const tq_status st = encode_args(cb, k, v, in_dtype, num_tokens, num_kv_heads, tok_stride, head_stride,
                                   slot_mapping, k_cache, v_cache, norms_out, a, &launch);
  if (st != TQ_OK || !launch) return st;
  hipError_t e = tq::launch_encode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "encode launch");
  return TQ_OK;
}

}  // extern "C"

namespace {
// Keys a sequence's walk covers at most: with a sliding window, from the
// page holding the first query's oldest key to the end.
int walk_span(int max_context_len, int q_len, int window) {
  if (window <= 0) return max_context_len;
  return (int)std::min<int64_t>(max_context_len, (int64_t)window + q_len - 1 + (tq::kBlock - 1));
}

// The fused decode step (append and query operands in one launch, then the
// split pass on the stream plan reading them, then the merge) serves 3-bit
// codes with up to 8 query heads per KV head and appends of at most
// kAppendMaxVectors vectors; other steps run the encode and the decode
// launches in turn.  A verify block of more than 8 query rows per KV head
// (G q_len, at most 32) runs the stream plan too, with a launch of its own
// for the query operands: one pass over the cache for every position, where
// the balanced plan's launches give each group of 8 / G positions a range of
// workgroups of its own.  (A single-query call keeps the balanced plan:
// without an append to share it with, the operands' launch costs more than
// the stream plan saves.)
bool step_fused(int bits, int q_len, int group, int num_seqs, int num_kv_heads, int64_t num_tokens) {
  return bits == 3 && q_len == 1 && group >= 1 && group <= 8 && tq::decode_uses_mfma(1, group, bits) &&
         num_tokens * num_kv_heads <= tq::kAppendMaxVectors && (int64_t)num_seqs * num_kv_heads <= 0x0fffffffLL;
}
constexpr int kVerifyStreamRows = 8;
bool verify_stream(int bits, int q_len, int group, int num_seqs, int num_kv_heads, int tokens_per_split,
                   int hot_parts) {
  return bits == 3 && q_len > 1 && tq::decode_uses_mfma(q_len, group, bits) && group * q_len > kVerifyStreamRows &&
         tokens_per_split == 0 && hot_parts == 0 && (int64_t)num_seqs * num_kv_heads <= 0x0fffffffLL;
}
// The stream plan: the tiles of all groups in one order, q consecutive tiles
// per run (1 <= q <= 16), one wave per run and head tile (P = ceil(R / 4)
// for the R = G q_len query rows of a group), q = ceil(P N / (4
// kStreamTarget)): at most max(4 kStreamTarget, N / 16) runs and P times as
// many waves, 4 per workgroup, the workgroups in one run per accelerator die
// (7 more cover the runs' rounding).  Each run writes a record per group it
// touches, at place (run + group): fewer than runs + groups places of R rows.
constexpr int kStreamTarget = 512;  // workgroups that fill the compute units once
int stream_pair(int rows) { return (rows + 3) / 4; }
int64_t stream_runs(int num_seqs, int num_kv_heads, int span) {
  const int64_t N = (int64_t)num_seqs * num_kv_heads * ((std::max(span, 0) + 127) / 128);
  return std::max<int64_t>(4 * kStreamTarget, (N + 15) / 16);
}
int64_t stream_grid(int num_seqs, int num_kv_heads, int rows, int span) {
  return (stream_pair(rows) * stream_runs(num_seqs, num_kv_heads, span) + 3) / 4 + 7;
}
size_t stream_record_floats(int num_seqs, int rows, int num_kv_heads, int span) {
  return (size_t)(stream_runs(num_seqs, num_kv_heads, span) + (int64_t)num_seqs * num_kv_heads) * rows * kPartStride;
}
// The stream plan's workspace: the records, then the query operands of each
// (group, head tile), then a descriptor per wave of the split pass's grid,
// then each group's (first record place, record count) for the merge.
size_t stream_qops_bytes(int num_seqs, int rows, int num_kv_heads) {
  return (size_t)num_seqs * num_kv_heads * stream_pair(rows) * tq::kQopsDwords * 64 * sizeof(uint32_t);
}
size_t stream_desc_bytes(int num_seqs, int rows, int num_kv_heads, int span) {
  return (size_t)stream_grid(num_seqs, num_kv_heads, rows, span) * 4 * tq::kDescWords * sizeof(uint32_t);
}
size_t step_workspace(int num_seqs, int q_len, int num_q_heads, int num_kv_heads, int span) {
  const int rows = num_q_heads / num_kv_heads * q_len;
  return stream_record_floats(num_seqs, rows, num_kv_heads, span) * sizeof(float) +
         stream_qops_bytes(num_seqs, rows, num_kv_heads) + stream_desc_bytes(num_seqs, rows, num_kv_heads, span) +
         (size_t)num_seqs * num_kv_heads * 2 * sizeof(int);  // the merge's (first place, records) per group
}

size_t decode_workspace(int bits, int num_seqs, int q_len, int num_q_heads, int num_kv_heads, int max_context_len,
                        int tokens_per_split, int hot_parts, int window = 0) {
  if (num_seqs < 1 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_context_len < 0 || window < 0)
    return 0;
  max_context_len = walk_span(max_context_len, q_len, window);
  const int grp = num_q_heads % num_kv_heads == 0 ? num_q_heads / num_kv_heads : 0;
  if (grp > 0 && verify_stream(bits, q_len, grp, num_seqs, num_kv_heads, tokens_per_split, hot_parts))
    return step_workspace(num_seqs, q_len, num_q_heads, num_kv_heads, max_context_len);
  const int ns = plan_splits(num_seqs, q_len, num_kv_heads, grp, max_context_len, tokens_per_split, bits).num_splits;
  const int64_t rows = (int64_t)num_seqs * q_len * num_q_heads;
  // the matrix-core split pass forms its query operands itself: partials only
  const bool mfma = grp > 0 && tq::decode_uses_mfma(q_len, grp, bits);
  const size_t words = (mfma ? 0 : tq::decode_qprep_floats(rows)) + tq::decode_partial_floats(rows, ns + hot_parts);
  return words * sizeof(float);
}

// Validation, planning and launch shared by the plain call and the call with
// an exact hot window (hot: non-null window arguments).
struct HotWindow {
  const void *k, *v;
  tq_dtype dtype;
  const int32_t *lens;
  int max;
};

tq_status decode_impl(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                      const uint8_t *k_cache, const uint8_t *v_cache,
                      const int32_t *block_tables, int max_blocks_per_seq,
                      const int32_t *context_lens, int num_seqs, int q_len,
                      int num_q_heads, int num_kv_heads, int max_context_len,
                      float softmax_scale, void *out, tq_dtype out_dtype,
                      int tokens_per_split, void *workspace, size_t workspace_bytes,
                      void *stream, const HotWindow *hot, bool noalloc = false, int window = 0,
                      const tq::EncodeArgs *step = nullptr) {
  tq_status st = check_cb(cb);
  if (st != TQ_OK) return st;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || (!workspace && !noalloc))
    return fail(TQ_ERR_INVALID_ARGUMENT, "null device pointer");
  if (!dtype_ok(q_dtype) || !dtype_ok(out_dtype)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (num_seqs < 1 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1)
    return fail(TQ_ERR_INVALID_ARGUMENT, "num_seqs, q_len and head counts must be >= 1");
  if (num_q_heads % num_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "num_q_heads (%d) not a multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  const int group = num_q_heads / num_kv_heads;
  if (group > tq::kMaxGroup) return fail(TQ_ERR_UNSUPPORTED, "more than %d query heads per KV head", tq::kMaxGroup);
  if (max_context_len < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "max_context_len < 0");
  if (q_len > 1 && q_len > max_context_len)
    return fail(TQ_ERR_INVALID_ARGUMENT, "q_len (%d) > max_context_len (%d)", q_len, max_context_len);
  if (window < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "window < 0");
  if (window > 0 && hot) return fail(TQ_ERR_UNSUPPORTED, "a sliding window does not combine with a hot window");
  if (max_blocks_per_seq < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "max_blocks_per_seq < 1");
  if (window == 0 && (int64_t)max_blocks_per_seq * tq::kBlock < max_context_len)
    return fail(TQ_ERR_INVALID_ARGUMENT, "max_blocks_per_seq (%d) cannot hold max_context_len (%d)",
                max_blocks_per_seq, max_context_len);
  // a ring of R pages holds 16 R consecutive positions: enough for the keys
  // of the whole query block (window + q_len - 1 positions)
  if (window > 0 && (int64_t)max_blocks_per_seq * tq::kBlock <
                        std::min<int64_t>(max_context_len, (int64_t)window + q_len - 1))
    return fail(TQ_ERR_INVALID_ARGUMENT,
                "a ring of %d pages cannot hold window (%d) + q_len (%d) - 1 positions", max_blocks_per_seq,
                window, q_len);
  const int span = walk_span(max_context_len, q_len, window);  // keys one sequence's walk covers
  if (tokens_per_split < 0 || (tokens_per_split > 0 && tokens_per_split % 256 != 0))
    return fail(TQ_ERR_INVALID_ARGUMENT, "tokens_per_split must be 0 or a positive multiple of 256");
  const int bits = cb->bits;
  if (tokens_per_split > tq::kMaxMfmaSplitTokens && tq::decode_uses_mfma(q_len, group, bits))
    return fail(TQ_ERR_UNSUPPORTED, "tokens_per_split %d exceeds the %d tokens per chunk of this pass",
                tokens_per_split, tq::kMaxMfmaSplitTokens);
  if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale))
    return fail(TQ_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if ((int64_t)num_seqs * q_len > 0x7fffffffLL) return fail(TQ_ERR_UNSUPPORTED, "num_seqs * q_len too large");
  const SplitPlan plan = plan_splits(num_seqs, q_len, num_kv_heads, group, span, tokens_per_split, bits);
  const int ns = plan.num_splits;
  if (ns > 65535) return fail(TQ_ERR_UNSUPPORTED, "too many splits (%d); raise tokens_per_split", ns);
  if ((int64_t)num_seqs * num_kv_heads * ((span + 127) / 128) > 0x7fffffffLL)
    return fail(TQ_ERR_UNSUPPORTED, "num_seqs * num_kv_heads * tiles of max_context_len too large");
  int hot_parts = 0;
  if (hot) {
    if (q_len != 1) return fail(TQ_ERR_UNSUPPORTED, "a hot window is supported for q_len == 1 only (got %d)", q_len);
    if (hot->max < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "hot_max < 0");
    if (!dtype_ok(hot->dtype)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown hot_dtype %d", (int)hot->dtype);
    if (hot->max > 0) {
      if (!hot->k || !hot->v || !hot->lens) return fail(TQ_ERR_INVALID_ARGUMENT, "null hot window pointer");
      if ((reinterpret_cast<uintptr_t>(hot->k) & 15) != 0 || (reinterpret_cast<uintptr_t>(hot->v) & 15) != 0)
        return fail(TQ_ERR_UNSUPPORTED, "hot_k and hot_v must be 16-byte aligned");
      if ((int64_t)num_seqs * hot->max * num_kv_heads > 0x7fffffffLL)
        return fail(TQ_ERR_UNSUPPORTED, "hot window too large");
    }
    hot_parts = tq::decode_hot_parts(hot->max);
    if (ns + hot_parts > 65535) return fail(TQ_ERR_UNSUPPORTED, "too many partial records per row");
  }
  const bool fused = step && step_fused(bits, q_len, group, num_seqs, num_kv_heads, step->num_tokens);
  const bool verify = !step && verify_stream(bits, q_len, group, num_seqs, num_kv_heads, tokens_per_split,
                                             hot_parts);
  if ((fused || verify) && (reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  const size_t need = fused || verify ? step_workspace(num_seqs, q_len, num_q_heads, num_kv_heads, span)
                            : decode_workspace(bits, num_seqs, q_len, num_q_heads, num_kv_heads, max_context_len,
                                               tokens_per_split, hot_parts, window);
  if (noalloc) {
    // every check above is on the host; the scratch array's address is
    // resolved (once per device) only for a call that will launch
    if (need > tq::kNoAllocScratchBytes)
      return fail(TQ_ERR_WORKSPACE_TOO_SMALL,
                  "the call needs %zu bytes of partial records, more than the %zu-byte device scratch of "
                  "tq_decode_attention_noalloc; use tq_decode_attention with a workspace",
                  need, (size_t)tq::kNoAllocScratchBytes);
    hipError_t e = tq::noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    workspace_bytes = tq::kNoAllocScratchBytes;
  }
  if (workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  tq::DecodeArgs a;
  a.q = q;
  a.q_dtype = q_dtype;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.q_len = q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.scale = softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / std::sqrt((double)tq::kHeadDim));
  a.out = out;
  a.out_dtype = out_dtype;
  a.split_tokens = plan.split_tokens;
  a.num_splits = ns;
  // a context length past the plan is cut to it (caller contract broken);
  // with a window the ring and the walk from seq_base bound every access
  a.window = window;
  if (window > 0)
    a.ctx_cap = max_context_len;
  else
    a.ctx_cap = plan.balanced ? std::min((int64_t)max_blocks_per_seq * tq::kBlock, (int64_t)max_context_len)
                              : (int)std::min((int64_t)max_blocks_per_seq * tq::kBlock, (int64_t)ns * plan.split_tokens);
  a.balanced = plan.balanced;
  a.bal_grid = plan.grid;
  a.bal_target = plan.target;
  a.bal_per = plan.per;
  a.bal_min = plan.min_tiles;
  a.St = (const float *)cb->d_tables + (size_t)tq::kQjlDim * tq::kHeadDim;
  a.SHop = (const uint16_t *)(a.St + (size_t)tq::kQjlDim * tq::kHeadDim);
  const int64_t rows = (int64_t)num_seqs * q_len * num_q_heads;
  a.qk_tiles = 0;
  a.pos0 = 0;
  a.pos_count = q_len;
  a.qprep = nullptr;
  float *rest = (float *)workspace;
  if (tq::decode_uses_mfma(q_len, group, bits)) {
    a.qk_tiles = tq::decode_qk_tiles(group * std::min(q_len, tq::decode_positions_per_launch(group)));
  } else {
    a.qprep = rest;
    rest += tq::decode_qprep_floats(rows);
  }
  a.partials = rest;
  a.part_stride = ns + hot_parts;
  a.hot_parts = hot_parts;
  a.hot_k = hot ? hot->k : nullptr;
  a.hot_v = hot ? hot->v : nullptr;
  a.hot_dtype = hot ? hot->dtype : TQ_F32;
  a.hot_lens = hot ? hot->lens : nullptr;
  a.hot_max = hot ? hot->max : 0;
  a.cb = device_codebook(cb);
  a.qops = nullptr;
  a.desc = nullptr;
  a.ginfo = nullptr;
  hipError_t e;
  if (fused || verify) {
    // stream plan: the records, then the operands (16-byte aligned: records of 528 bytes)
    const int64_t grid = stream_grid(num_seqs, num_kv_heads, group * q_len, span);
    // the first launch: the append's workgroups, one per (group, head tile), one per split workgroup
    const int64_t first = (fused ? (step->num_tokens * num_kv_heads + tq::kAppendWaves - 1) / tq::kAppendWaves : 0) +
                          (int64_t)num_seqs * num_kv_heads * stream_pair(group * q_len) + grid;
    if (grid > 0x7fffffffLL || first > 0x7fffffffLL) return fail(TQ_ERR_UNSUPPORTED, "too many tiles for one launch");
    a.balanced = 2;
    a.bal_target = kStreamTarget;
    a.bal_grid = (int)grid;
    a.partials = (float *)workspace;
    a.qops = reinterpret_cast<uint32_t *>(a.partials +
                                          stream_record_floats(num_seqs, group * q_len, num_kv_heads, span));
    a.desc = a.qops + stream_qops_bytes(num_seqs, group * q_len, num_kv_heads) / sizeof(uint32_t);
    a.ginfo = reinterpret_cast<int2 *>(a.desc + stream_desc_bytes(num_seqs, group * q_len, num_kv_heads, span) /
                                                   sizeof(uint32_t));
    e = tq::launch_step_prep(fused ? step : nullptr, a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fused ? "decode step launch" : "verify operands launch");
  } else if (step) {
    e = tq::launch_encode(*step, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "encode launch");
  }
  e = tq::launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return TQ_OK;
}
}  // namespace

extern "C" {

size_t tq_decode_workspace_bytes(const tq_codebook *cb, int num_seqs, int q_len,
                                 int num_q_heads, int num_kv_heads, int max_context_len,
                                 int tokens_per_split) {

  return decode_workspace(cb_bits(cb), num_seqs, q_len, num_q_heads, num_kv_heads, max_context_len,
                          tokens_per_split, 0);
}

tq_status tq_decode_attention(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                              const uint8_t *k_cache, const uint8_t *v_cache,
                              const int32_t *block_tables, int max_blocks_per_seq,
                              const int32_t *context_lens, int num_seqs, int q_len,
                              int num_q_heads, int num_kv_heads, int max_context_len,
                              float softmax_scale, void *out, tq_dtype out_dtype,
                              int tokens_per_split, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return decode_impl(cb, q, q_dtype, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, q_len, num_q_heads, num_kv_heads, max_context_len, softmax_scale, out,
                     out_dtype, tokens_per_split, workspace, workspace_bytes, stream, nullptr);
}

tq_status tq_decode_attention_noalloc(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                                      const uint8_t *k_cache, const uint8_t *v_cache,
                                      const int32_t *block_tables, int max_blocks_per_seq,
                                      const int32_t *context_lens, int num_seqs, int q_len,
                                      int num_q_heads, int num_kv_heads, int max_context_len,
                                      float softmax_scale, void *out, tq_dtype out_dtype,
                                      int tokens_per_split, void *stream) {
  return decode_impl(cb, q, q_dtype, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, q_len, num_q_heads, num_kv_heads, max_context_len, softmax_scale, out,
                     out_dtype, tokens_per_split, nullptr, 0, stream, nullptr, true);
}

size_t tq_decode_noalloc_scratch_bytes(void) { return tq::kNoAllocScratchBytes; }

size_t tq_decode_window_workspace_bytes(const tq_codebook *cb, int num_seqs, int q_len, int num_q_heads,
                                        int num_kv_heads, int max_context_len, int window,
                                        int tokens_per_split) {

  if (window < 1) return 0;
  return decode_workspace(cb_bits(cb), num_seqs, q_len, num_q_heads, num_kv_heads, max_context_len, tokens_per_split, 0,
                          window);
}

tq_status tq_decode_attention_window(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                                     const uint8_t *k_cache, const uint8_t *v_cache,
                                     const int32_t *block_tables, int ring_blocks,
                                     const int32_t *context_lens, int num_seqs, int q_len,
                                     int num_q_heads, int num_kv_heads, int max_context_len, int window,
                                     float softmax_scale, void *out, tq_dtype out_dtype,
                                     int tokens_per_split, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  if (window < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "window must be >= 1 (got %d)", window);
  return decode_impl(cb, q, q_dtype, k_cache, v_cache, block_tables, ring_blocks, context_lens, num_seqs,
                     q_len, num_q_heads, num_kv_heads, max_context_len, softmax_scale, out, out_dtype,
                     tokens_per_split, workspace, workspace_bytes, stream, nullptr, false, window);
}

size_t tq_decode_hot_workspace_bytes(const tq_codebook *cb, int num_seqs, int num_q_heads,
                                     int num_kv_heads, int max_context_len, int hot_max,
                                     int tokens_per_split) {

  if (hot_max < 0) return 0;
  return decode_workspace(cb_bits(cb), num_seqs, 1, num_q_heads, num_kv_heads, max_context_len, tokens_per_split,
                          tq::decode_hot_parts(hot_max));
}

size_t tq_decode_step_workspace_bytes(const tq_codebook *cb, int num_seqs, int num_q_heads, int num_kv_heads,
                                      int max_context_len, int tokens_per_split) {
  const int bits = cb_bits(cb);
  const size_t need =
      decode_workspace(bits, num_seqs, 1, num_q_heads, num_kv_heads, max_context_len, tokens_per_split, 0);
  if (need == 0 || num_q_heads % num_kv_heads != 0) return need;
  const int group = num_q_heads / num_kv_heads;
  if (step_fused(bits, 1, group, num_seqs, num_kv_heads, num_seqs))
    return step_workspace(num_seqs, 1, num_q_heads, num_kv_heads, max_context_len);
  return need;
}

tq_status tq_decode_step(const tq_codebook *cb, const void *k_new, const void *v_new, tq_dtype kv_dtype,
                         int64_t tok_stride, int64_t head_stride, const int64_t *slot_mapping, const void *q,
                         tq_dtype q_dtype, uint8_t *k_cache, uint8_t *v_cache, const int32_t *block_tables,
                         int max_blocks_per_seq, const int32_t *context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int max_context_len, float softmax_scale, void *out, tq_dtype out_dtype,
                         int tokens_per_split, void *workspace, size_t workspace_bytes, void *stream) {
  if (num_seqs < 1) return fail(TQ_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
  tq::EncodeArgs ea;
  bool launch;
  const tq_status st = encode_args(cb, k_new, v_new, kv_dtype, num_seqs, num_kv_heads, tok_stride, head_stride,
                                   slot_mapping, k_cache, v_cache, nullptr, ea, &launch);
  if (st != TQ_OK) return st;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return decode_impl(cb, q, q_dtype, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, 1,
                     num_q_heads, num_kv_heads, max_context_len, softmax_scale, out, out_dtype, tokens_per_split,
                     workspace, workspace_bytes, stream, nullptr, false, 0, &ea);
}

tq_status tq_decode_attention_hot(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                                  const uint8_t *k_cache, const uint8_t *v_cache,
                                  const int32_t *block_tables, int max_blocks_per_seq,
                                  const int32_t *context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int max_context_len, const void *hot_k,
                                  const void *hot_v, tq_dtype hot_dtype, const int32_t *hot_lens,
                                  int hot_max, float softmax_scale, void *out, tq_dtype out_dtype,
                                  int tokens_per_split, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  const HotWindow hw{hot_k, hot_v, hot_dtype, hot_lens, hot_max};
  return decode_impl(cb, q, q_dtype, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, 1, num_q_heads, num_kv_heads, max_context_len, softmax_scale, out,
                     out_dtype, tokens_per_split, workspace, workspace_bytes, stream, &hw);
}

}  // extern "C"
