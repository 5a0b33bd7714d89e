/*
 * tq.h -- C ABI of libtq: TurboQuant KV-cache compression and attention read
 * directly from the compressed, paged cache, on AMD Instinct MI355X (gfx950).
 *
 * The method (sources: SwiftLM README, section "TurboQuantization: KV Cache
 * Compression"; lilting.ch SwiftLM article, sections "Lloyd-Maxコードブックとは",
 * "KVキャッシュ圧縮の内訳" and "Walsh-Hadamard Transform（WHT）の役割"; 0h-n0
 * vLLM-MLX explainer, section "Paged KVキャッシュ"):
 *   key   (4.25 bits/coordinate): norm -> normalise -> Walsh-Hadamard rotation
 *         -> 3-bit Lloyd-Max code per coordinate for N(0, 1/d) -> residual
 *         against the quantised vector -> 1-bit signs of a random Gaussian
 *         (QJL) projection of that residual;
 *   value (3.125 bits/coordinate): the same without the QJL stage.
 *
 * Conventions for every entry point:
 *   - All functions return tq_status; nothing throws across the ABI.  On a
 *     non-OK status tq_last_error() returns a thread-local message.
 *   - Arguments are checked on the host before anything is launched; a
 *     rejected call launches nothing and leaves every buffer untouched.
 *   - Device pointers are plain HIP device addresses owned by the caller.
 *     The library never allocates, frees or synchronises in the encode and
 *     attention calls; work is enqueued on the caller's HIP stream
 *     (hipStream_t passed as void*, NULL = default stream) and is complete
 *     when that stream is.
 *   - Only head_dim = 128, qjl_dim = 128, 2-, 3- or 4-bit codes and 16-token
 *     blocks are supported; other values give TQ_ERR_UNSUPPORTED.  3 bits
 *     (the pages' method) decode on the matrix-core passes, 2 and 4 bits on
 *     the vector pass.
 *   - Not checked (caller contract): block-table entries lie inside the
 *     pools, context lengths cover only slots that were encoded, and
 *     slot_mapping holds no duplicate slot.
 *
 * Page layout (little-endian; bit b of a byte has weight 2^b), one page per
 * (block, KV head), pools k_cache[num_blocks][num_kv_heads][tq_k_page_bytes]
 * and v_cache[num_blocks][num_kv_heads][tq_v_page_bytes], slot = block * 16 +
 * offset.  For b-bit codes (b = cb->bits; 3 in the pages' method) and
 * RB = 4 (b + 1) bytes per record:
 *   K page (256 (b + 1) + 64 bytes; 1088 for b = 3):
 *           [0, 64 RB): 64 records of RB bytes, record (chunk g, token t) at
 *           RB (16 g + t) for g = 0..3; its 32-bit word f = 0 .. b-1 holds
 *           bit-plane f of the codes of coordinates 32g .. 32g+31
 *           (coordinate 32g + k at bit k), word b the QJL sign bits of
 *           projection rows 32g .. 32g+31 (1 = projection >= 0);
 *           [64 RB, 64 RB + 32): half norm of token t at 64 RB + 2t;
 *           [64 RB + 32, 64 RB + 64): half residual length gamma.
 *   V page (256 b + 32 bytes; 800 for b = 3): [256p, 256p+256), p < b:
 *           bit-plane p, coordinate-major: coordinate i owns the 16-bit word
 *           at 256p + 2i, token t at its bit t; [256 b, 256 b + 32): half
 *           norm of token t at 256 b + 2t.
 *   Code value = rank of the codebook level in ascending order.
 *   b = 3: 1088*8/(16*128) = 4.25 and 800*8/(16*128) = 3.125 bits per
 *   coordinate; b = 2: 3.25 and 2.125; b = 4: 5.25 and 4.125.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARGUMENT = -1,   /* null pointer, negative size, bad stride ... */
  TQ_ERR_UNSUPPORTED = -2,        /* valid but not implemented (e.g. head_dim != 128) */
  TQ_ERR_WORKSPACE_TOO_SMALL = -3,
  TQ_ERR_NOT_INITIALIZED = -4,    /* codebook not set up by tq_codebook_init */
  TQ_ERR_HIP = -5                 /* a HIP runtime call failed; see tq_last_error() */
} tq_status;

typedef enum tq_dtype { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 } tq_dtype;

#define TQ_HEAD_DIM 128
#define TQ_QJL_DIM 128
#define TQ_BITS 3
#define TQ_BLOCK 16
#define TQ_K_PAGE_BYTES 1088
#define TQ_V_PAGE_BYTES 800

/* Codebook and projection context.  Caller-owned storage, filled by
 * tq_codebook_init and read-only afterwards; several threads and streams may
 * share one.  d_tables points at the caller's device buffer of
 * tq_codebook_device_bytes() bytes, which must outlive every call using it. */
typedef struct tq_codebook {
  int32_t head_dim;        /* 128 */
  int32_t bits;            /* 2, 3 or 4 (the pages' method: 3) */
  int32_t qjl_dim;         /* 128 */
  int32_t block_size;      /* 16 */
  uint64_t qjl_seed;       /* seed of the generated S (0 if caller-supplied) */
  float centroids[16];     /* ascending fp32 levels for N(0, 1/d); 2^bits used */
  float thresholds[15];    /* fp32 midpoints of adjacent levels; 2^bits - 1 used */
  float qjl_scale;         /* sqrt(pi/2) / qjl_dim */
  void *d_tables;          /* device, 16-byte aligned: S [m][d] fp32, S^T [d][m] fp32,
                              then S*H as half pairs (hi, lo = S*H - hi) in an
                              internal order (2*m*d halves) */
  uint32_t magic;          /* set by tq_codebook_init */
  uint32_t reserved;
} tq_codebook;

/* ---- host-only helpers (no device needed) ------------------------------ */

/* Lloyd-Max codebook for N(0, 1/head_dim) with 2^bits levels (lilting.ch
 * article, "Lloyd-Maxコードブックとは"): the fixed point of "thresholds are
 * midpoints, levels are conditional means", iterated in double precision on
 * N(0,1), scaled by 1/sqrt(head_dim) and rounded once to fp32.  Writes
 * 2^bits levels and 2^bits - 1 thresholds, ascending.  bits in [1, 4]. */
tq_status tq_codebook_compute(int head_dim, int bits, float *centroids, float *thresholds);

/* QJL matrix S (rows x cols, fp32, row-major) from a seed: SplitMix64
 * (Steele, Lea, Flood 2014) uniforms u = ((x >> 11) + 0.5) * 2^-53, pairs
 * turned into normals by Box-Muller in double (r cos, r sin), row-major fill,
 * one rounding to fp32.  The SwiftLM README ("TurboQuantization", K-cache
 * step 5) names a random Johnson-Lindenstrauss projection; this generator is
 * this library's fixed choice so results are reproducible from the seed. */
tq_status tq_qjl_matrix(uint64_t seed, int rows, int cols, float *out);

/* ---- context ------------------------------------------------------------ */

/* Bytes of the device table buffer for a codebook of this size. */
size_t tq_codebook_device_bytes(int head_dim, int qjl_dim);

/* Fill *cb (host struct) and upload [S | S^T | S*H halves] to d_tables on
 * `stream`, then wait for `stream` (a one-time set-up call; it is the only
 * call that copies host data to the device or synchronises).
 * qjl_host: NULL -> S generated from qjl_seed by tq_qjl_matrix; else the
 * caller's S (qjl_dim x head_dim fp32 row-major host array).
 * bits 2, 3 or 4 (3 is the pages' method and runs on the matrix-core passes;
 * 2 and 4 are codebook variants whose decode runs on the vector pass).
 * Errors: TQ_ERR_UNSUPPORTED for head_dim/qjl_dim other than 128/128 or bits
 * outside 2..4,
 * TQ_ERR_INVALID_ARGUMENT for null cb/d_tables or d_tables not 16-byte
 * aligned, TQ_ERR_HIP on copy failure. */
tq_status tq_codebook_init(tq_codebook *cb, int head_dim, int bits, uint64_t qjl_seed,
                           const float *qjl_host, void *d_tables, void *stream);

size_t tq_k_page_bytes(const tq_codebook *cb);   /* 256 (bits + 1) + 64: 1088 for 3 bits */
size_t tq_v_page_bytes(const tq_codebook *cb);   /* 256 bits + 32: 800 for 3 bits */

/* ---- encode --------------------------------------------------------------
 * Compress num_tokens x num_kv_heads key and value vectors and store each
 * (token, head) record in its slot (SwiftLM README, "TurboQuantization",
 * K-cache steps 1-5 and the V-cache paragraph; paging per the vLLM-MLX
 * explainer, "Paged KVキャッシュ").
 *   k, v        device, element (t, h, i) at k[t*tok_stride + h*head_stride + i]
 *               (strides in elements; i contiguous), dtype in_dtype; both
 *               16-byte aligned with strides that are multiples of 8 elements
 *               (4 for fp32), else TQ_ERR_UNSUPPORTED.
 *   slot_mapping device int64[num_tokens]; a negative slot skips the token.
 *   k_cache, v_cache device pools as laid out above.
 *   norms_out   nullable device fp32[num_tokens][num_kv_heads][3]: the fp32
 *               |k|, gamma and |v| the encoder computed (before rounding to
 *               half), for checking; skipped tokens are left untouched.
 * num_tokens == 0 is a no-op.  Decision thresholds are compared in fp32. */
tq_status tq_encode_kv(const tq_codebook *cb, const void *k, const void *v, tq_dtype in_dtype,
                       int64_t num_tokens, int num_kv_heads, int64_t tok_stride,
                       int64_t head_stride, const int64_t *slot_mapping, uint8_t *k_cache,
                       uint8_t *v_cache, float *norms_out, void *stream);

/* ---- attention ------------------------------------------------------------
 * out[b][t][h] = sum_j softmax_j(scale * <q[b][t][h], k~_j>) v~_j over the
 * compressed keys/values of sequence b and KV head h / (Hq/Hkv), where
 * k~ = |k| (H^T c[idx] + sqrt(pi/2)/m * gamma * S^T sigma) and
 * v~ = |v| H^T c[idx_v] -- the QJL-corrected inner-product estimate of the
 * SwiftLM README's K-cache step 5, attention over the whole compressed
 * history (its note on --turbo-kv recall) read through a block table.
 * q_len > 1 (chunked prefill, the README's --prefill-size, or a block of
 * tokens to verify in speculative multi-token decoding, the README's "MTP
 * Speculative Decoding" performance section) is causal: query t sees keys
 * 0 .. context_len - q_len + t.
 *   q           device [num_seqs][q_len][num_q_heads][128], dtype q_dtype.
 *   block_tables device int32[num_seqs][max_blocks_per_seq].
 *   context_lens device int32[num_seqs], each in [0, max_context_len]; the
 *               length includes the q_len new tokens.  0 gives zero output.
 *   softmax_scale 0 -> 1/sqrt(128).
 *   out         device [num_seqs][q_len][num_q_heads][128], dtype out_dtype.
 *   tokens_per_split  0 -> chosen by the library; else a multiple of 256
 *               giving the split-K chunk (results agree to rounding).
 *               Decode with up to 8 query heads per KV head and a short
 *               query block (at most 4 groups of 8 / group positions) uses
 *               at most 8192 tokens per chunk.
 *   workspace   device scratch of tq_decode_workspace_bytes() bytes (same
 *               arguments); contents on entry do not matter.  16-byte
 *               aligned for a verify block of 9 to 32 query rows per KV
 *               head (q_len x Hq / Hkv, with tokens_per_split 0), whose
 *               query operands the library forms in a launch of their own
 *               and keeps in the workspace.
 * Any group size num_q_heads / num_kv_heads from 1 to 16 is accepted.
 * Errors: TQ_ERR_INVALID_ARGUMENT (nulls, Hq % Hkv != 0, q_len < 1,
 * q_len > max_context_len, bad tokens_per_split, a misaligned workspace
 * where alignment is required), TQ_ERR_UNSUPPORTED
 * (num_q_heads / num_kv_heads > 16, tokens_per_split above 8192 where the
 * chunk limit above applies, or a batch whose launches would need 2^31 or
 * more workgroups), TQ_ERR_WORKSPACE_TOO_SMALL. */
size_t tq_decode_workspace_bytes(const tq_codebook *cb, int num_seqs, int q_len,
                                 int num_q_heads, int num_kv_heads, int max_context_len,
                                 int tokens_per_split);

tq_status tq_decode_attention(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                              const uint8_t *k_cache, const uint8_t *v_cache,
                              const int32_t *block_tables, int max_blocks_per_seq,
                              const int32_t *context_lens, int num_seqs, int q_len,
                              int num_q_heads, int num_kv_heads, int max_context_len,
                              float softmax_scale, void *out, tq_dtype out_dtype,
                              int tokens_per_split, void *workspace, size_t workspace_bytes,
                              void *stream);

/* ---- attention without a caller workspace ----------------------------------
 * For callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results as tq_decode_attention, minus the
 * workspace: its partial records go to a device scratch array inside the
 * library (one per device, tq_decode_noalloc_scratch_bytes() = 64 MiB, held
 * until the process ends; its address on a device is resolved by
 * tq_codebook_init on the current device, or by the first call on another).
 * The call allocates and frees nothing.  All calls on one device share that
 * array: calls that overlap on a device (several streams or threads) race
 * and must be serialised by the caller.
 * Errors: those of tq_decode_attention; TQ_ERR_WORKSPACE_TOO_SMALL when the
 * call's partial records (tq_decode_workspace_bytes() for the same
 * arguments) exceed the scratch size; TQ_ERR_HIP if the scratch address
 * cannot be resolved. */
size_t tq_decode_noalloc_scratch_bytes(void);

tq_status tq_decode_attention_noalloc(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                                      const uint8_t *k_cache, const uint8_t *v_cache,
                                      const int32_t *block_tables, int max_blocks_per_seq,
                                      const int32_t *context_lens, int num_seqs, int q_len,
                                      int num_q_heads, int num_kv_heads, int max_context_len,
                                      float softmax_scale, void *out, tq_dtype out_dtype,
                                      int tokens_per_split, void *stream);

/* ---- attention with an exact hot window -----------------------------------
 * The SwiftLM README keeps the recent tokens uncompressed and compresses only
 * past a threshold (its --turbo-kv option row: after 2,048 tokens), and
 * attention covers both (its note on --turbo-kv long-range recall).  This
 * call is tq_decode_attention for one new token per sequence (q_len = 1)
 * whose keys are the context_lens[b] compressed tokens of the paged cache
 * followed by hot_lens[b] exact tokens: one softmax over all of them.
 *   hot_k, hot_v device [num_seqs][hot_max][num_kv_heads][128], dtype
 *               hot_dtype, 16-byte aligned (token j of sequence b, KV head h
 *               at ((b * hot_max + j) * num_kv_heads + h) * 128).
 *   hot_lens    device int32[num_seqs], each in [0, hot_max] (values outside
 *               are cut to that range).  hot_max == 0: no window; the
 *               pointers may then be NULL.
 *   workspace   tq_decode_hot_workspace_bytes() bytes (same arguments).
 * The other arguments are those of tq_decode_attention with q_len = 1 (the
 * query is [num_seqs][1][num_q_heads][128]; context_lens may be 0).
 * A sequence with no key at all gets a zero output.
 * Errors: those of tq_decode_attention, TQ_ERR_INVALID_ARGUMENT (hot_max < 0,
 * null window pointers with hot_max > 0, unknown hot_dtype),
 * TQ_ERR_UNSUPPORTED (misaligned window, window too large). */
size_t tq_decode_hot_workspace_bytes(const tq_codebook *cb, int num_seqs, int num_q_heads,
                                     int num_kv_heads, int max_context_len, int hot_max,
                                     int tokens_per_split);

tq_status tq_decode_attention_hot(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                                  const uint8_t *k_cache, const uint8_t *v_cache,
                                  const int32_t *block_tables, int max_blocks_per_seq,
                                  const int32_t *context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int max_context_len, const void *hot_k,
                                  const void *hot_v, tq_dtype hot_dtype, const int32_t *hot_lens,
                                  int hot_max, float softmax_scale, void *out, tq_dtype out_dtype,
                                  int tokens_per_split, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* ---- sliding-window attention over a rotating cache -----------------------
 * Sliding-window layers keep only their most recent tokens; the SwiftLM
 * README ("Performance: Mac mini M6", the correction under its tables and the
 * --turbo-kv recall note) points out that such layers run on a rotating
 * cache (Gemma 4: 25 of 30 layers with a 1,024-token window) which its
 * compression did not cover.  This call is tq_decode_attention where
 *   - query t of sequence b (position p = context_lens[b] - q_len + t) sees
 *     only the keys at positions max(0, p - window + 1) .. p;
 *   - block_tables row b is a ring of ring_blocks pages: position j lives in
 *     page block_tables[b][(j / 16) mod ring_blocks] at offset j % 16, so a
 *     page is reused for the positions 16 ring_blocks later (the caller's
 *     slot_mapping for tq_encode_kv follows the same rule; a ring with
 *     16 ring_blocks >= max_context_len never wraps and is a plain table).
 * The ring must hold the keys of the whole query block:
 * 16 ring_blocks >= min(max_context_len, window + q_len - 1); the call then
 * reads only the pages the windows overlap (about window + q_len - 1 + 15
 * positions per sequence, whatever the context length).
 *   window      >= 1.
 *   workspace   tq_decode_window_workspace_bytes() bytes (same arguments).
 * Other arguments as in tq_decode_attention (ring_blocks in the place of
 * max_blocks_per_seq).  Errors: those of tq_decode_attention, and
 * TQ_ERR_INVALID_ARGUMENT for window < 1 or a ring too small. */
size_t tq_decode_window_workspace_bytes(const tq_codebook *cb, int num_seqs, int q_len, int num_q_heads,
                                        int num_kv_heads, int max_context_len, int window,
                                        int tokens_per_split);

tq_status tq_decode_attention_window(const tq_codebook *cb, const void *q, tq_dtype q_dtype,
                                     const uint8_t *k_cache, const uint8_t *v_cache,
                                     const int32_t *block_tables, int ring_blocks,
                                     const int32_t *context_lens, int num_seqs, int q_len,
                                     int num_q_heads, int num_kv_heads, int max_context_len, int window,
                                     float softmax_scale, void *out, tq_dtype out_dtype,
                                     int tokens_per_split, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* ---- one decode step: append, then attend ---------------------------------
 * A generation step compresses the new token's key and value into the cache
 * and then attends over the whole compressed history with its query (the
 * SwiftLM README, "TurboQuantization: KV Cache Compression": the K-cache
 * steps 1-5 at write time, the step-5 estimate at read time; paging per the
 * vLLM-MLX explainer, "Paged KVキャッシュ").  This call is exactly
 *   tq_encode_kv(cb, k_new, v_new, kv_dtype, num_seqs, num_kv_heads,
 *                tok_stride, head_stride, slot_mapping, k_cache, v_cache,
 *                NULL, stream)
 * followed by tq_decode_attention(..., q_len = 1, ...) with the remaining
 * arguments, on `stream`: the cache contents are bit-identical to those two
 * calls'.  With 3-bit codes, up to 8 query heads per KV head and at most
 * 1,024 new (token, KV head) vectors it runs fused, in three launches
 * instead of four: the append shares its launch with the attention's
 * per-(sequence, KV head) query set-up, and the split pass gives every wave
 * an equal share of all the batch's tiles (tokens_per_split is not used);
 * the output then equals the two calls' up to the rounding of the softmax
 * combine (fp32 with up to 4 heads per KV head; with 5 to 8, within the
 * weights' 15-bit rounding, since the separate call then runs another
 * split pass).  Otherwise it runs the two calls' launches and the output
 * is bit-identical.
 *   k_new, v_new  device, element (b, h, i) of sequence b's new token at
 *               k_new[b*tok_stride + h*head_stride + i], as in tq_encode_kv.
 *   slot_mapping device int64[num_seqs]: the slot of sequence b's new token
 *               (negative: no append for b).
 *   context_lens include the new token.
 *   workspace   tq_decode_step_workspace_bytes() bytes (same arguments),
 *               16-byte aligned.
 * Other arguments as in tq_decode_attention with q_len = 1.  Errors: those
 * of tq_encode_kv and tq_decode_attention, TQ_ERR_INVALID_ARGUMENT for a
 * misaligned workspace; on an error nothing is launched. */
size_t tq_decode_step_workspace_bytes(const tq_codebook *cb, int num_seqs, int num_q_heads, int num_kv_heads,
                                      int max_context_len, int tokens_per_split);

tq_status tq_decode_step(const tq_codebook *cb, const void *k_new, const void *v_new, tq_dtype kv_dtype,
                         int64_t tok_stride, int64_t head_stride, const int64_t *slot_mapping, const void *q,
                         tq_dtype q_dtype, uint8_t *k_cache, uint8_t *v_cache, const int32_t *block_tables,
                         int max_blocks_per_seq, const int32_t *context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int max_context_len, float softmax_scale, void *out, tq_dtype out_dtype,
                         int tokens_per_split, void *workspace, size_t workspace_bytes, void *stream);

/* Thread-local text describing the last non-OK status on this thread. */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
