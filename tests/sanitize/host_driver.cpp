// Drives the host side of libkvq (argument validation, tables, record sizes, the cache planner's
// bookkeeping and truncation) with no device present, for a build of kvq_host.cpp with the
// address and undefined-behaviour sanitizers (tests/test_host_sanitizers.py). Every call here
// returns before anything is enqueued; device pointers are fake, 16-byte-aligned addresses that
// are never dereferenced. Exit status 0 = every expectation held and no sanitizer finding.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/kvq.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "expectation failed at line %d: %s (last error: %s)\n", \
                   __LINE__, #cond, kvq_last_error());                            \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

static void* fake(uintptr_t k) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + 4096 * k); }

static kvq_codec codec(uint32_t D, uint32_t bits) {
  kvq_codec c;
  std::memset(&c, 0, sizeof c);
  c.head_dim = D;
  c.bits = bits;
  c.seed = 42 + D;
  return c;
}

int main() {
  EXPECT(kvq_abi_version() == KVQ_ABI_VERSION);
  // record sizes and tables for every valid shape; refusals for invalid ones
  const uint32_t dims[] = {64, 128, 256, 512};
  for (uint32_t D : dims)
    for (uint32_t b = 1; b <= 4; ++b) {
      kvq_codec c = codec(D, b);
      EXPECT(kvq_record_bytes(&c) == D * b / 8 + 4);
      float cen[16], thr[15];
      int8_t sg[512];
      EXPECT(kvq_codec_tables(&c, cen, thr, sg) == KVQ_OK);
      for (uint32_t k = 1; k < (1u << b); ++k) EXPECT(cen[k] > cen[k - 1]);
      c.outlier_T = 2.0f;
      EXPECT(kvq_encode_workspace_bytes(&c, 100000) > 0);
      EXPECT(kvq_fit_workspace_bytes(&c, 4096) > 0 || D == 0);
    }
  {
    kvq_codec c = codec(96, 3);
    EXPECT(kvq_record_bytes(&c) == 0);
    c = codec(128, 5);
    EXPECT(kvq_record_bytes(&c) == 0);
    c = codec(128, 3);
    c.flags = 7;
    EXPECT(kvq_encode(&c, fake(1), 4, 128, fake(2), nullptr, nullptr, nullptr) == KVQ_E_ARG);
    const float bad[4] = {0.0f, -1.0f, 1.0f, 2.0f};
    c = codec(128, 2);
    c.centroids_host = bad;
    EXPECT(kvq_encode(&c, fake(1), 4, 128, fake(2), nullptr, nullptr, nullptr) == KVQ_E_CENTROIDS);
    c = codec(128, 3);
    c.proj_rank = 48;
    EXPECT(kvq_record_bytes(&c) == 0);
  }
  // argument refusals of every device call
  {
    kvq_codec c = codec(128, 3);
    EXPECT(kvq_encode(&c, nullptr, 4, 128, fake(2), nullptr, nullptr, nullptr) == KVQ_E_NULL);
    EXPECT(kvq_encode(&c, fake(1), 4, 100, fake(2), nullptr, nullptr, nullptr) == KVQ_E_STRIDE);
    EXPECT(kvq_encode(&c, fake(1), -1, 128, fake(2), nullptr, nullptr, nullptr) != KVQ_OK);
    EXPECT(kvq_decode(&c, nullptr, 4, nullptr, fake(3), KVQ_BF16, 128, nullptr) == KVQ_E_NULL);
    EXPECT(kvq_decode(&c, fake(2), 4, nullptr, fake(3), KVQ_BF16, 100, nullptr) == KVQ_E_STRIDE);
    EXPECT(kvq_score_packed(&c, fake(1), 2, 12, 12 * 128, 128, fake(2), 5, 64, 5 * 64, 64,
                            static_cast<float*>(fake(3)), 12 * 64, 64, nullptr) != KVQ_OK);
    EXPECT(kvq_score_packed(&c, nullptr, 2, 8, 8 * 128, 128, fake(2), 2, 64, 2 * 64, 64,
                            static_cast<float*>(fake(3)), 8 * 64, 64, nullptr) == KVQ_E_NULL);
    kvq_codec v = codec(128, 2);
    EXPECT(kvq_attend_workspace_bytes(&v, 2, 2, 4096) > 0);
    EXPECT(kvq_attend_packed(&c, &v, fake(1), 2, 8, 8 * 128, 128, fake(2), fake(3), 2, 0, 2 * 64,
                             64, 0.1f, 0.0f, static_cast<float*>(fake(4)), 8 * 128, 128, fake(5),
                             1 << 20, nullptr) != KVQ_OK);  // T = 0 is refused
    EXPECT(kvq_attend_packed_static(&c, &v, fake(1), 1024, 8, 8 * 128, 128, fake(2), fake(3), 1,
                                    64, 64, 64, 0.1f, 0.0f, static_cast<float*>(fake(4)), 8 * 128,
                                    128, nullptr) == KVQ_E_CAPACITY);
    float cen[8];
    EXPECT(kvq_fit_table(&c, fake(1), 0, 128, 3, cen, fake(2), 1 << 20, nullptr) != KVQ_OK);
    EXPECT(kvq_fit_table(&c, fake(1), 1024, 128, -1, cen, fake(2), 1 << 20, nullptr) == KVQ_E_ARG);
    uint32_t sink = 0;
    EXPECT(kvq_stream_copy(fake(1), fake(2), 24, nullptr) == KVQ_E_ARG);
    EXPECT(kvq_stream_read(nullptr, 32, &sink, nullptr) == KVQ_E_NULL);
    EXPECT(kvq_stream_fill(fake(1), 20, 7, nullptr) == KVQ_E_ARG);
    EXPECT(std::strlen(kvq_last_error()) > 0);
  }
  // caches: init, refusals, and truncation bookkeeping (host only)
  {
    kvq_codec c = codec(128, 3);
    kvq_cache cache;
    std::memset(&cache, 0, sizeof cache);
    EXPECT(kvq_cache_init(&c, &cache, fake(10), 4096, fake(11), 1024, 256, 16) == KVQ_OK);
    EXPECT(cache.packed_len == 0 && cache.tail_len == 0);
    EXPECT(kvq_cache_truncate(&c, &cache, 0) == KVQ_OK);
    EXPECT(kvq_cache_truncate(&c, &cache, 1) == KVQ_E_ARG);
    kvq_codec other = codec(128, 2);
    EXPECT(kvq_cache_truncate(&other, &cache, 0) == KVQ_E_CACHE);
    kvq_cache forged;
    std::memset(&forged, 0, sizeof forged);
    EXPECT(kvq_cache_truncate(&c, &forged, 0) == KVQ_E_CACHE);
    // a cache whose lengths the planner would have set: truncation maps them onto both regions
    cache.packed_len = 512;
    cache.tail_len = 300;
    cache.tail_head = 1000;
    EXPECT(kvq_cache_truncate(&c, &cache, 700) == KVQ_OK);
    EXPECT(cache.packed_len == 512 && cache.tail_len == 188);
    EXPECT(kvq_cache_truncate(&c, &cache, 100) == KVQ_OK);
    EXPECT(cache.packed_len == 100 && cache.tail_len == 0);
    EXPECT(kvq_cache_truncate(&c, &cache, 101) == KVQ_E_ARG);
    EXPECT(kvq_cache_init(&c, &cache, fake(10), -1, fake(11), 1024, 256, 16) != KVQ_OK);
    EXPECT(kvq_cache_init(&c, &cache, fake(10), 4096, nullptr, 1024, 256, 16) == KVQ_E_NULL);
    kvq_cache* list[1] = {&forged};
    const void* rows[1] = {fake(12)};
    int64_t evicted[1] = {0};
    EXPECT(kvq_append_evict_chunk(&c, list, 1, rows, 1, nullptr, evicted) == KVQ_E_CACHE);
  }
  if (failures) return 1;
  std::printf("host driver ok\n");
  return 0;
}
