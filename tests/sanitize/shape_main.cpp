// Drives the library's host shape logic (paged_attention_quantized_kv_amd/csrc/shape.cpp) over
// ordinary and extreme arguments, built with the address and undefined-behaviour sanitizers
// by tests/test_sanitize.py: every call must return without a sanitizer report, supported
// shapes must satisfy the chunking invariants, and out-of-range ones must be refused.
#include <stdio.h>
#include <stdlib.h>

#include <climits>
#include <vector>

#include "../../paged_attention_quantized_kv_amd/csrc/shape.h"

static int fails = 0;
#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);     \
      ++fails;                                                         \
    }                                                                  \
  } while (0)

int main() {
  const int Bs[] = {1, 2, 3, 8, 31, 32, 33, 64, 1023, 1024, 1025, 0, -1, INT_MAX};
  const int Ts[] = {1, 4, 8, 9, 0, -3};
  const int heads[][2] = {{24, 4}, {8, 1}, {32, 4}, {64, 2}, {8, 3}, {65535, 65535}, {1, 0}, {INT_MAX, 1}};
  const int Ds[] = {128, 256, 64, 0};
  const int Ls[] = {1, 63, 64, 65, 2048, 32768, 131072, 262144, 1 << 24, INT_MAX, 0, -5};
  long supported = 0;
  for (int B : Bs)
    for (int T : Ts)
      for (auto &h : heads)
        for (int D : Ds)
          for (int L : Ls) {
            kvq::AttnShape s;
            const int rc = kvq::attn_shape(B, T, h[0], h[1], D, L, &s);
            if (rc != KVQ_OK) {
              CHECK(rc == KVQ_ERR_INVALID_ARG || rc == KVQ_ERR_UNSUPPORTED);
              continue;
            }
            ++supported;
            CHECK(s.tokens_per_split % kvq::kPage == 0 && s.tokens_per_split > 0);
            CHECK(static_cast<long>(s.n_splits) * s.tokens_per_split >= L);
            CHECK(static_cast<long>(s.n_splits - 1) * s.tokens_per_split < L);
            CHECK(s.rows == T * (h[0] / h[1]));
            CHECK(s.slots >= (s.balanced ? kvq::kTargetWgs : 1));
            CHECK(s.ml_bytes >= static_cast<size_t>(s.slots) * s.rows * 8 && s.ml_bytes % 256 == 0);
            CHECK(s.o_bytes == static_cast<size_t>(s.slots) * s.rows * D * 4);
            for (int rows_blk : {64, 128}) {
              kvq::PrefillShape p;
              const int rp = kvq::prefill_shape(B, T, h[0], h[1], D, L, rows_blk, &p);
              if (rp != KVQ_OK) continue;
              CHECK(static_cast<long>(p.row_blocks) * rows_blk >= p.rows);
              CHECK(static_cast<long>(p.n_splits) * p.tokens_per_split >= L);
              CHECK(p.direct == (p.n_splits == 1));
            }
          }
  // prefill with very long chunks of rows
  for (int T : {1, 4096, 1 << 20, INT_MAX}) {
    kvq::PrefillShape p;
    const int rc = kvq::prefill_shape(1, T, 24, 4, 256, T > 262144 ? INT_MAX : 262144, 128, &p);
    CHECK(rc == KVQ_OK || rc == KVQ_ERR_UNSUPPORTED || rc == KVQ_ERR_INVALID_ARG);
  }
  // page-pool descriptors
  std::vector<unsigned char> buf(4096 + 64);
  unsigned char *al = buf.data() + (16 - reinterpret_cast<uintptr_t>(buf.data()) % 16) % 16;
  kvq_cache_t c = {KVQ_INT8_G64, 8, 64, 4, 256, 0, al, al + 256, al + 512, al + 768};
  CHECK(kvq::check_cache(&c) == KVQ_OK);
  CHECK(kvq::check_cache(nullptr) == KVQ_ERR_INVALID_ARG);
  kvq_cache_t bad = c;
  bad.k_codes = al + 1;
  CHECK(kvq::check_cache(&bad) == KVQ_ERR_INVALID_ARG);
  bad = c;
  bad.format = 9;
  CHECK(kvq::check_cache(&bad) == KVQ_ERR_INVALID_ARG);
  bad = c;
  bad.block_size = 32;
  CHECK(kvq::check_cache(&bad) == KVQ_ERR_UNSUPPORTED);
  bad = c;
  bad.format = KVQ_BF16_KV;
  bad.k_scales = bad.v_scales = nullptr;
  CHECK(kvq::check_cache(&bad) == KVQ_OK);
  for (int L : {1, 64, 1 << 20, INT_MAX}) CHECK(kvq::chunk_tokens(1, 4, L) % kvq::kPage == 0);
  // contexts beyond 2^30 tokens are refused (the kernels count tokens and pages in 32 bits)
  {
    kvq::AttnShape s;
    kvq::PrefillShape p;
    CHECK(kvq::attn_shape(1, 1, 8, 1, 128, kvq::kMaxSeqLen, &s) == KVQ_OK);
    CHECK(kvq::attn_shape(1, 1, 8, 1, 128, kvq::kMaxSeqLen + 1, &s) == KVQ_ERR_UNSUPPORTED);
    CHECK(kvq::prefill_shape(1, 1, 8, 1, 128, kvq::kMaxSeqLen, 64, &p) == KVQ_OK);
    CHECK(kvq::prefill_shape(1, 1, 8, 1, 128, kvq::kMaxSeqLen + 1, 64, &p) == KVQ_ERR_UNSUPPORTED);
  }
  CHECK(kvq::balanced_slots(32, 8, INT_MAX) > kvq::kTargetWgs);
  // capacity planning over extreme lengths and pool sizes
  {
    int64_t deficit = -1;
    std::vector<int32_t> lens = {0, 1, 64, 65, kvq::kMaxSeqLen, INT_MAX, -1};
    for (int fmt = 0; fmt <= 5; ++fmt)
      for (int D : {64, 128, 256}) CHECK(kvq::page_bytes(fmt, D) % 64 == 0);
    for (int32_t nblk : {1, 1000, INT_MAX}) {
      kvq_cache_t cc = c;
      cc.num_blocks = nblk;
      cc.num_kv_heads = 65535;
      for (size_t i = 0; i < lens.size(); ++i) {
        const int rc = kvq::capacity_check(&cc, 1, &lens[i], 1, &deficit);
        CHECK(rc == KVQ_OK || rc == KVQ_ERR_CAPACITY || rc == KVQ_ERR_INVALID_ARG || rc == KVQ_ERR_UNSUPPORTED);
        CHECK(deficit >= 0);
      }
      std::vector<int32_t> many(1 << 12, kvq::kMaxSeqLen);
      const int rc = kvq::capacity_check(&cc, static_cast<int32_t>(many.size()), many.data(), INT_MAX, &deficit);
      CHECK((rc == KVQ_OK) == (deficit == 0) && deficit >= 0);
    }
    CHECK(kvq::capacity_check(&c, 1, nullptr, 1, &deficit) == KVQ_ERR_INVALID_ARG);
    CHECK(kvq::capacity_check(&c, 1, &lens[0], 1, nullptr) == KVQ_ERR_INVALID_ARG);
  }
  printf("shape logic: %ld supported shapes checked, %d failures\n", supported, fails);
  if (fails == 0) printf("shape ok\n");
  return fails == 0 ? 0 : 1;
}
