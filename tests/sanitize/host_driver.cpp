// Host-only driver of the C ABI for the AddressSanitizer / UndefinedBehavior-
// Sanitizer build: codebook and projection generation, every size query over
// a sweep of shapes (plan arithmetic near its limits), and the argument
// checks of every call that fail before any device work.  Prints
// "host driver ok" when every expectation holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "tq.h"

static int failures = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static void *const FAKE = reinterpret_cast<void *>(uintptr_t{1} << 40);

static tq_codebook fake_cb(int bits) {
  tq_codebook c;
  std::memset(&c, 0, sizeof c);
  c.head_dim = 128;
  c.bits = bits;
  c.qjl_dim = 128;
  c.block_size = 16;
  c.d_tables = FAKE;
  c.magic = 0x54513031u;
  return c;
}

int main() {
  // codebooks: ascending, odd-symmetric levels; thresholds between levels
  for (int bits = 1; bits <= 4; ++bits) {
    float c[16], t[15];
    EXPECT(tq_codebook_compute(128, bits, c, t) == TQ_OK);
    const int n = 1 << bits;
    for (int i = 0; i < n; ++i) EXPECT(std::fabs(c[i] + c[n - 1 - i]) < 1e-7f);
    for (int i = 0; i + 1 < n; ++i) EXPECT(c[i] < t[i] && t[i] < c[i + 1]);
  }
  float c[16], t[15];
  EXPECT(tq_codebook_compute(128, 5, c, t) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_codebook_compute(128, 3, nullptr, t) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(std::strlen(tq_last_error()) > 0);

  std::vector<float> S(128 * 128);
  EXPECT(tq_qjl_matrix(42, 128, 128, S.data()) == TQ_OK);
  double s2 = 0.0;
  for (float x : S) s2 += (double)x * x;
  EXPECT(std::fabs(s2 / S.size() - 1.0) < 0.05);
  EXPECT(tq_qjl_matrix(42, 0, 128, S.data()) != TQ_OK);
  EXPECT(tq_codebook_device_bytes(128, 128) > 0);

  tq_codebook init;
  std::memset(&init, 0, sizeof init);
  EXPECT(tq_codebook_init(&init, 64, 3, 1, nullptr, FAKE, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_codebook_init(&init, 128, 5, 1, nullptr, FAKE, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_codebook_init(&init, 128, 3, 1, nullptr, nullptr, nullptr) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(tq_codebook_init(nullptr, 128, 3, 1, nullptr, FAKE, nullptr) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(init.magic == 0);

  // size queries over a sweep of shapes, up to the limits of the plan
  const int seqs[] = {1, 3, 16, 1000, 1 << 20};
  const int ctxs[] = {0, 1, 127, 128, 8192, 131072, 1 << 24, 1 << 30};
  const int qls[] = {1, 2, 3, 8, 21, 2048};
  const int heads[][2] = {{32, 8}, {32, 4}, {32, 2}, {28, 4}, {16, 16}, {64, 2}};
  for (int bits = 2; bits <= 4; ++bits) {
    tq_codebook cb = fake_cb(bits);
    EXPECT(tq_k_page_bytes(&cb) == (size_t)(256 * (bits + 1) + 64));
    EXPECT(tq_v_page_bytes(&cb) == (size_t)(256 * bits + 32));
    for (int B : seqs)
      for (int L : ctxs)
        for (int ql : qls)
          for (auto &hh : heads)
            for (int tps : {0, 256, 8192}) {
              (void)tq_decode_workspace_bytes(&cb, B, ql, hh[0], hh[1], L, tps);
              (void)tq_decode_window_workspace_bytes(&cb, B, ql, hh[0], hh[1], L, 1024, tps);
              if (ql == 1) {
                (void)tq_decode_hot_workspace_bytes(&cb, B, hh[0], hh[1], L, 2048, tps);
                (void)tq_decode_step_workspace_bytes(&cb, B, hh[0], hh[1], L, tps);
              }
            }
  }
  EXPECT(tq_decode_workspace_bytes(nullptr, 0, 1, 32, 8, 100, 0) == 0);
  EXPECT(tq_decode_window_workspace_bytes(nullptr, 4, 1, 32, 8, 100, 0, 0) == 0);

  // argument checks that end before any device work
  tq_codebook cb = fake_cb(3), raw = fake_cb(3);
  raw.magic = 0;
  const uint8_t *kc = static_cast<const uint8_t *>(FAKE);
  const int32_t *ip = static_cast<const int32_t *>(FAKE);
  auto dec = [&](const tq_codebook *k, const void *q, int B, int ql, int hq, int hkv, int mb, int maxc, int tps,
                 size_t wsb) {
    return tq_decode_attention(k, q, TQ_BF16, kc, kc, ip, mb, ip, B, ql, hq, hkv, maxc, 0.0f, FAKE, TQ_F32, tps,
                               FAKE, wsb, nullptr);
  };
  EXPECT(dec(&raw, FAKE, 1, 1, 32, 8, 64, 1024, 0, 1ull << 40) == TQ_ERR_NOT_INITIALIZED);
  EXPECT(dec(&cb, nullptr, 1, 1, 32, 8, 64, 1024, 0, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(dec(&cb, FAKE, 0, 1, 32, 8, 64, 1024, 0, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(dec(&cb, FAKE, 1, 1, 30, 8, 64, 1024, 0, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(dec(&cb, FAKE, 1, 1, 64, 2, 64, 1024, 0, 1ull << 40) == TQ_ERR_UNSUPPORTED);
  EXPECT(dec(&cb, FAKE, 1, 1, 32, 8, 63, 1024, 0, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(dec(&cb, FAKE, 1, 1, 32, 8, 64, 1024, 100, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(dec(&cb, FAKE, 1, 1, 32, 8, 1024, 16384, 16384, 1ull << 40) == TQ_ERR_UNSUPPORTED);
  EXPECT(dec(&cb, FAKE, 1, 1, 32, 8, 64, 1024, 0, 16) == TQ_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(dec(&cb, FAKE, 1 << 20, 2048, 32, 8, 1 << 20, 1 << 24, 0, 1ull << 40) != TQ_OK);
  EXPECT(tq_decode_attention_noalloc(&cb, FAKE, TQ_BF16, kc, kc, ip, 1 << 16, ip, 256, 1, 32, 8, 1 << 20, 0.0f, FAKE,
                                     TQ_F32, 0, nullptr) == TQ_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(tq_decode_attention_window(&cb, FAKE, TQ_BF16, kc, kc, ip, 70, ip, 1, 1, 32, 8, 100000, 0, 0.0f, FAKE, TQ_F32,
                                    0, FAKE, 1ull << 40, nullptr) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(tq_decode_attention_window(&cb, FAKE, TQ_BF16, kc, kc, ip, 63, ip, 1, 1, 32, 8, 100000, 1024, 0.0f, FAKE,
                                    TQ_F32, 0, FAKE, 1ull << 40, nullptr) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(tq_decode_attention_hot(&cb, FAKE, TQ_BF16, kc, kc, ip, 64, ip, 1, 32, 8, 1024, FAKE, FAKE, TQ_BF16, ip, -1,
                                 0.0f, FAKE, TQ_F32, 0, FAKE, 1ull << 40, nullptr) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(tq_encode_kv(&cb, FAKE, FAKE, TQ_BF16, -1, 8, 1024, 128, static_cast<const int64_t *>(FAKE),
                      static_cast<uint8_t *>(FAKE), static_cast<uint8_t *>(FAKE), nullptr, nullptr) ==
         TQ_ERR_INVALID_ARGUMENT);
  EXPECT(tq_encode_kv(&cb, FAKE, FAKE, TQ_BF16, 4, 8, 1024, 100, static_cast<const int64_t *>(FAKE),
                      static_cast<uint8_t *>(FAKE), static_cast<uint8_t *>(FAKE), nullptr, nullptr) != TQ_OK);
  auto step = [&](const void *k, int B, int hq, int hkv, int mb, int maxc, const void *ws, size_t wsb) {
    return tq_decode_step(&cb, k, k, TQ_BF16, 1024, 128, static_cast<const int64_t *>(FAKE), FAKE, TQ_BF16,
                          static_cast<uint8_t *>(FAKE), static_cast<uint8_t *>(FAKE), ip, mb, ip, B, hq, hkv, maxc,
                          0.0f, FAKE, TQ_F32, 0, const_cast<void *>(ws), wsb, nullptr);
  };
  EXPECT(step(nullptr, 1, 32, 8, 64, 1024, FAKE, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(step(FAKE, 0, 32, 8, 64, 1024, FAKE, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(step(FAKE, 1, 32, 8, 64, 1024, static_cast<const char *>(FAKE) + 8, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(step(FAKE, 1, 32, 8, 63, 1024, FAKE, 1ull << 40) == TQ_ERR_INVALID_ARGUMENT);
  EXPECT(step(FAKE, 16, 32, 8, 2048, 32768, FAKE, 16) == TQ_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(step(FAKE, 1 << 20, 32, 8, 1 << 20, 1 << 24, FAKE, 1ull << 40) != TQ_OK);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host driver ok\n");
  return 0;
}
