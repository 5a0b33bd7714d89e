// Internal interface between the C-ABI host layer (tq_host.cpp) and the HIP
// kernels (tq_encode.hip, tq_decode.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kHeadDim = 128;
constexpr int kQjlDim = 128;
constexpr int kBlock = 16;
constexpr int kKPage = 1088;
constexpr int kVPage = 800;
constexpr int kMaxGroup = 16;       // query heads per KV head handled by one workgroup
constexpr int kAppendWaves = 4;     // appended vectors (one per wave) per workgroup of the step's first launch
constexpr uint32_t kMagic = 0x54513031u;  // "TQ01"

// Offsets inside a K page / V page (see tq.h).  K page: 64 records of 16
// bytes, record (chunk g, token t) at 16 (16 g + t) holding the 32-bit words
// of code bit-planes 0, 1, 2 and of the QJL signs for coordinates (rows)
// 32 g .. 32 g + 31; then the half norms and residual lengths.  V page: three
// coordinate-major bit-planes of 256 bytes, then the half norms.
constexpr int kKRecords = 1024;     // bytes of 16-byte (chunk, token) records
constexpr int kKSignField = 3;      // word of a record holding the QJL signs
constexpr int kKNorm = 1024;
constexpr int kKGamma = 1056;
constexpr int kVPlane = 256;        // bytes per V code bit-plane
constexpr int kVNorm = 768;
// Byte offset of the record of coordinate chunk g, token t of a K page.
constexpr int k_record(int g, int t) { return 16 * (16 * g + t); }

// Page geometry for b-bit codes (b = 2, 3, 4): K records of b code-plane
// words and one sign word per (32-coordinate chunk, token), then the halves
// n and gamma; V pages of b coordinate-major planes, then n.
constexpr int k_rec_bytes(int b) { return 4 * (b + 1); }
constexpr int k_norm_off(int b) { return 64 * k_rec_bytes(b); }
constexpr int k_page_bytes(int b) { return k_norm_off(b) + 64; }
constexpr int v_norm_off(int b) { return 256 * b; }
constexpr int v_page_bytes(int b) { return v_norm_off(b) + 32; }
static_assert(k_page_bytes(3) == kKPage && v_page_bytes(3) == kVPage && k_norm_off(3) == kKNorm &&
                  v_norm_off(3) == kVNorm, "3-bit geometry");

struct Codebook {
  float c[16];       // ascending levels (2^bits used)
  float t[15];       // thresholds (2^bits - 1 used)
  int bits;          // 2, 3 or 4
  float qjl_scale;   // sqrt(pi/2)/m
  // Bit-plane form of the levels: with B_p = 1 - 2 b_p for the code bits
  // b0, b1, b2 and their xor, c[idx] = -(beta0 B0 + beta1 B1 + beta2 B2 + beta3 Bx)
  // exactly (the levels are an odd function of the bits: c[7-i] = -c[i]).
  float beta[4];
};

struct EncodeArgs {
  const void *k;
  const void *v;
  int dtype;
  int64_t num_tokens;
  int num_kv_heads;
  int64_t tok_stride;
  int64_t head_stride;
  const int64_t *slots;
  uint8_t *k_cache;
  uint8_t *v_cache;
  float *norms_out;
  const float *S;    // [m][d]
  const float *St;   // [d][m]
  const uint16_t *SHop;  // half bits of S H (hi, lo) in the encoder's operand order
  Codebook cb;
};

struct DecodeArgs {
  const void *q;
  int q_dtype;
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const int32_t *block_tables;
  int max_blocks;
  const int32_t *context_lens;
  int num_seqs;
  int q_len;
  int num_q_heads;
  int num_kv_heads;
  int window;          // > 0: query at position p sees keys p - window + 1 .. p, and the
                       // block-table row is a ring (logical page P at entry P mod max_blocks)
  int group;           // num_q_heads / num_kv_heads
  float scale;
  void *out;
  int out_dtype;
  int split_tokens;
  int num_splits;
  // Context lengths are cut to ctx_cap (what the block table row and the
  // plan of partial records cover).
  int ctx_cap;
  // Balanced plan of the matrix-core decode pass (balanced = 1): the tiles
  // of 128 tokens of every (sequence, KV head) group are cut into ranges of
  // `per` tiles, one workgroup each, numbered densely sequence-major then
  // head-major; per = bal_per if > 0, else the smallest multiple of 4 in
  // [bal_min, 64] whose ranges number at most bal_target (or 64), computed
  // on the device from the context lengths.  Range j of a group writes the
  // group's partial record j.  The grid has bal_grid workgroups, enough for
  // every range.
  int balanced;
  int bal_grid, bal_target, bal_per, bal_min;
  const float *St;     // [d][m]
  const uint16_t *SHop;  // S H as f16 hi, lo halves in the projection's operand order
  float *qprep;        // workspace (vector and prefill passes): [rows][256] = rotated q | qjl_scale * S q
  // Matrix-core split pass: it forms its own query operands, for the
  // positions pos0 .. pos0 + pos_count - 1 of the q_len new ones (at most 8
  // query rows, positions x heads, per KV head and launch; several launches
  // cover more positions), in qk_tiles 16-row operand tiles (4 rows x 4
  // digits each); qk_tiles is 0 for the other passes.
  int qk_tiles;
  int pos0, pos_count;
  float *partials;     // workspace: [rows][part_stride][4 + 128], m in log2 units
  // Partial records per row: the num_splits chunks of the compressed cache,
  // then (for a call with an exact hot window) hot_parts chunks of
  // kHotChunk window tokens, placed right after the row's visible chunks.
  int part_stride;
  int hot_parts;
  const void *hot_k;   // [num_seqs][hot_max][num_kv_heads][128], dtype hot_dtype
  const void *hot_v;
  int hot_dtype;
  const int32_t *hot_lens;  // [num_seqs], cut to [0, hot_max]
  int hot_max;
  // The fused decode step (balanced = 2, the stream plan: the tiles of all
  // groups in one order, an equal share per wave, one record per (wave,
  // group) at place wave + group, G rows each; partials then hold those
  // places): qops holds each (sequence, KV head) group's matrix operands,
  // kQopsDwords per lane (null otherwise).
  uint32_t *qops;
  // The stream plan's per-wave descriptors (one per wave of the split pass's
  // grid, kDescWords each), formed in the operands launch: the wave's block
  // ids, tile slots and run, so the split pass starts on its pages at once.
  uint32_t *desc;
  // and each (sequence, KV head) group's first record place and record
  // count (x, y), formed in the same launch for the merge
  int2 *ginfo;
  Codebook cb;
};
constexpr int kQopsDwords = 44;  // per lane: 5 fp6 operands of 6 dwords, 5 scales, 2 x 4 start values, 1 pad
constexpr int kDescWords = 256;  // per wave: ids0 [64] | ids1 [64] | 16 slots x 4 | (tiles, run, head tile, 0) | pad

constexpr int kHotChunk = 64;  // exact window tokens per partial record
// Largest chunk of the matrix-core decode pass (64 tiles of 128 tokens).
constexpr int kMaxMfmaSplitTokens = 8192;

// Workspace split of tq_decode_attention.
size_t decode_qprep_floats(int64_t rows);
size_t decode_partial_floats(int64_t rows, int parts);
int decode_hot_parts(int hot_max);
// The matrix-core split pass serves decode with up to 8 heads per KV head
// and short query blocks (multi-token verify), one launch per group of
// 8 / group positions, at most 4 launches; single-query decode with 16 heads
// per KV head uses the vector pass, longer query blocks the prefill pass.
bool decode_uses_mfma(int q_len, int group, int bits);
int decode_positions_per_launch(int group);
// Several queries per sequence (chunked prefill, causal) run on the
// matrix-core prefill pass: 128 query rows (128 / group positions) per
// workgroup.
constexpr int64_t kAppendMaxVectors = 1024;  // encode calls of at most this many (token, KV head) vectors take one wave each
constexpr int kPrefillRows = 128;  // query rows (positions x heads) per prefill workgroup
bool prefill_uses_mfma(int q_len, int group, int bits);
int prefill_block_queries(int group);
int decode_qk_tiles(int rows);

// Device scratch of tq_decode_attention_noalloc: a file-scope __device__
// array (one copy per device, held until the process ends).  noalloc_scratch
// returns its address on the current device, resolved with
// hipGetSymbolAddress on the first request per device and kept; ptr may be
// null to resolve only.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// The stream plan's query operands launch (3-bit codes; the split pass then
// runs the stream plan), with the fused decode step's append in the same
// launch (ea non-null; q_len 1, up to 8 query heads per KV head) or alone
// (a verify block of up to 32 query rows per KV head).
hipError_t launch_step_prep(const EncodeArgs *ea, const DecodeArgs &a, hipStream_t stream);
hipError_t launch_prefill(const DecodeArgs &a, hipStream_t stream);

}  // namespace tq
