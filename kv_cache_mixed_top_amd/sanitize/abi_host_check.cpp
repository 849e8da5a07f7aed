// Host-side checks of the C ABI (include/semkv.h), built from every library
// source with the host compiler's AddressSanitizer and UndefinedBehavior-
// Sanitizer (kv_cache_mixed_top_amd/sanitize.py).  It runs with no visible
// GPU: every argument check, size query and launch plan runs on the host,
// and a call that gets as far as a launch returns SEMKV_EHIP instead of
// touching a device.  The pointers below are never dereferenced on the host.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "semkv.h"

static int failures = 0;

#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

static semkv_geom geom(int32_t batch = 1, int32_t Lh = 6, int32_t Ll = 5, int64_t ch = 16384,
                       int64_t cl = 16384, int32_t rotate = 0) {
  semkv_geom g;
  std::memset(&g, 0, sizeof g);
  g.batch = batch;
  g.layers = 32;
  g.kv_heads = 8;
  g.q_heads = 32;
  g.head_dim = 128;
  g.L_high = Lh;
  g.L_low = Ll;
  g.block = 128;
  g.cap_high = ch;
  g.cap_low = cl;
  g.rotate = rotate;
  return g;
}

static semkv_cache cache(const semkv_geom& g) {
  semkv_cache c;
  std::memset(&c, 0, sizeof c);
  c.g = g;
  c.codes_high = static_cast<uint8_t*>(P(0x10000000));
  c.codes_low = static_cast<uint8_t*>(P(0x20000000));
  c.meta_high = static_cast<uint16_t*>(P(0x30000000));
  c.meta_low = static_cast<uint16_t*>(P(0x40000000));
  c.tok_high = static_cast<int32_t*>(P(0x50000000));
  c.tok_low = static_cast<int32_t*>(P(0x60000000));
  c.tail_kv = static_cast<uint16_t*>(P(0x70000000));
  c.tail_score = static_cast<float*>(P(0x80000000));
  return c;
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::fprintf(stderr, "a GPU is visible: this check must run with none\n");
    return 2;
  }
  // sizes
  EXPECT(semkv_row_bytes(6) == 43 && semkv_row_bytes(5) == 38 && semkv_row_bytes(3) == 26);
  EXPECT(semkv_row_bytes(8) == 48 && semkv_row_bytes(16) == 64 && semkv_row_bytes(65536) == 256);
  for (int L = 3; L <= 70000; L += (L < 300 ? 1 : 997)) {
    const int64_t R = semkv_row_bytes(L);
    EXPECT(L > 65536 ? R < 0 : (R >= 26 && R <= 256));
  }
  EXPECT(semkv_row_bytes(2) < 0);
  EXPECT(semkv_topr_count(32768, 0.5) == 16384 && semkv_topr_count(300, 0.25) == 75);
  EXPECT(semkv_topr_count(-1, 0.5) < 0 && semkv_topr_count(10, 1.5) < 0);

  semkv_geom g = geom();
  int64_t sz[8];
  EXPECT(semkv_cache_sizes(&g, sz) == SEMKV_OK);
  EXPECT(sz[0] == (int64_t)1 * 32 * 8 * 2 * 16384 * 43);
  EXPECT(semkv_cache_sizes(nullptr, sz) == SEMKV_EINVAL);
  semkv_geom bad = g;
  bad.cap_high = 100;                                         // not a multiple of 16
  EXPECT(semkv_cache_sizes(&bad, sz) == SEMKV_EINVAL);
  bad = g;
  bad.head_dim = 64;
  EXPECT(semkv_cache_sizes(&bad, sz) == SEMKV_EUNSUPPORTED);
  bad = g;
  bad.L_low = 7;                                              // L_low > L_high
  EXPECT(semkv_cache_sizes(&bad, sz) == SEMKV_EINVAL);
  const int64_t ws = semkv_workspace_bytes(&g, 32, 32768);
  EXPECT(ws > 0);
  EXPECT(semkv_workspace_bytes(&g, 33, 10) < 0);

  // rank
  EXPECT(semkv_rank_topr(nullptr, 1, 100, 100, 10, static_cast<int32_t*>(P(0x1000)), nullptr, nullptr) ==
         SEMKV_EINVAL);
  EXPECT(semkv_rank_topr(static_cast<float*>(P(0x1000)), 1, 100, 100, 101, static_cast<int32_t*>(P(0x2000)),
                         nullptr, nullptr) == SEMKV_EINVAL);
  EXPECT(semkv_rank_topr(static_cast<float*>(P(0x1000)), 1, 100, 99, 10, static_cast<int32_t*>(P(0x2000)),
                         nullptr, nullptr) == SEMKV_EINVAL);
  // a valid call reaches the launch, which fails without a device
  EXPECT(semkv_rank_topr(static_cast<float*>(P(0x1000)), 1, 100, 100, 10, static_cast<int32_t*>(P(0x2000)),
                         nullptr, nullptr) == SEMKV_EHIP);

  // quantize-pack
  semkv_cache c = cache(g);
  const int64_t st[4] = {32LL * 8 * 32768 * 128, 8LL * 32768 * 128, 32768LL * 128, 128};
  const uint16_t* kv = static_cast<const uint16_t*>(P(0x90000000));
  const int32_t* perm = static_cast<const int32_t*>(P(0xA0000000));
  EXPECT(semkv_quantize_pack(&c, kv, kv, st, 32768, perm, 16385, nullptr) == SEMKV_ECAPACITY);
  EXPECT(semkv_quantize_pack(&c, kv, kv, st, 32768, perm, 32769, nullptr) == SEMKV_EINVAL);
  EXPECT(semkv_quantize_pack(&c, nullptr, kv, st, 32768, perm, 16384, nullptr) == SEMKV_EINVAL);
  EXPECT(semkv_quantize_pack(&c, kv, kv, st, 32768, perm, 16384, nullptr) == SEMKV_EHIP);
  EXPECT(c.n_high == 0 && c.n_low == 0);                       // nothing advanced on failure

  // decode: every level pair and query group plans its launch
  const int32_t pairs[][2] = {{6, 5}, {5, 4}, {4, 3}, {8, 6}, {16, 16}, {65536, 7}, {255, 100}};
  for (const auto& pr : pairs) {
    for (int32_t qh : {8, 16, 32, 64}) {
      for (int32_t rot : {0, 1}) {
        semkv_geom gd = geom(2, pr[0], pr[1], 4096, 4096, rot);
        gd.q_heads = qh;
        semkv_cache cd = cache(gd);
        cd.n_high = 4000;
        cd.n_low = 3000;
        cd.n_tail = 100;
        cd.n_tokens = 7100;
        const int64_t w = semkv_workspace_bytes(&gd, 32, 7100);
        EXPECT(w > 0);
        const uint16_t* q = static_cast<const uint16_t*>(P(0xB0000000));
        float* out = static_cast<float*>(P(0xC0000000));
        EXPECT(semkv_decode_attn(&cd, q, 0, 32, 1.0f, out, P(0xD0000000), w, nullptr) == SEMKV_EHIP);
        EXPECT(semkv_decode_attn(&cd, q, 0, 32, 1.0f, out, P(0xD0000000), 16, nullptr) == SEMKV_EWORKSPACE);
        EXPECT(semkv_decode_attn(&cd, q, 31, 2, 1.0f, out, P(0xD0000000), w, nullptr) == SEMKV_EINVAL);
        EXPECT(semkv_decode_attn_noalloc(&cd, q, 0, 32, 1.0f, out, nullptr) == SEMKV_EHIP);
        EXPECT(semkv_ragged_decode_attn(&cd, static_cast<const int64_t*>(P(0xE0000000)), q, 0, 32, 1.0f,
                                        4000, 3000, out, P(0xD0000000), w, nullptr) == SEMKV_EINVAL);
      }
    }
  }

  // generation
  semkv_cache cg = cache(geom());
  EXPECT(semkv_append_block(&cg, kv, kv, st, static_cast<const float*>(P(0xF0000000)), 1, 0.25, 0,
                            P(0xD0000000), 16, nullptr) == SEMKV_EWORKSPACE);
  EXPECT(semkv_append_block(&cg, kv, kv, st, static_cast<const float*>(P(0xF0000000)), 1, 1.5, 0,
                            P(0xD0000000), 1 << 20, nullptr) == SEMKV_EINVAL);
  semkv_cache full = cache(geom(1, 6, 5, 16, 16));
  EXPECT(semkv_append_block(&full, kv, kv, st, static_cast<const float*>(P(0xF0000000)), 128, 0.25, 0,
                            P(0xD0000000), 1 << 20, nullptr) == SEMKV_ECAPACITY);

  // ragged batches
  int64_t* seq = static_cast<int64_t*>(P(0xE0000000));
  const int32_t* nseq = static_cast<const int32_t*>(P(0xE1000000));
  EXPECT(semkv_seq_reset(nullptr, 2, nullptr) == SEMKV_EINVAL);
  EXPECT(semkv_seq_reset(seq, 2, nullptr) == SEMKV_EHIP);
  EXPECT(semkv_ragged_quantize_pack(&c, nullptr, kv, kv, st, 100, nseq, 0.5, perm, nullptr) == SEMKV_EINVAL);
  EXPECT(semkv_ragged_quantize_pack(&c, seq, kv, kv, st, 100, nseq, 0.5, perm, nullptr) == SEMKV_EHIP);
  EXPECT(semkv_ragged_append(&c, seq, kv, kv, st, static_cast<const float*>(P(0xF0000000)),
                             nseq, nullptr, 0.5, P(0xD0000000), 16, nullptr) == SEMKV_EWORKSPACE);
  EXPECT(semkv_ragged_decode_attn(&c, seq, static_cast<const uint16_t*>(P(0xB0000000)), 0, 32, 1.0f,
                                  16384, 16384, static_cast<float*>(P(0xC0000000)), P(0xD0000000),
                                  semkv_workspace_bytes(&g, 32, 32768 + 128), nullptr) == SEMKV_EHIP);

  // scoring
  const int64_t hs[3] = {5LL * 1000 * 4096, 1000LL * 4096, 4096};
  EXPECT(semkv_score_hidden_delta(kv, hs, 1, 5, 1000, 4096, static_cast<float*>(P(0x1000)), 1000, nullptr) ==
         SEMKV_EHIP);
  EXPECT(semkv_score_hidden_delta(kv, hs, 1, 10, 1000, 4096, static_cast<float*>(P(0x1000)), 1000, nullptr) ==
         SEMKV_EINVAL);
  EXPECT(semkv_score_keynorm(kv, st, 1, 8, 1000, 28, 4, static_cast<float*>(P(0x1000)), 1000, nullptr) ==
         SEMKV_EHIP);

  for (int s = -5; s <= 0; ++s) EXPECT(semkv_status_str(s) != nullptr);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
