// Drives the host library (validation, planner, plan description, the host-side checks of
// every entry point) over a seeded sweep of valid and invalid problems. Built with the
// address and undefined-behaviour sanitizers by tests/test_sanitize_host.py; any report
// aborts the program. Prints "ok <problems>" at the end.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../decode_attention_verify_amd/csrc/internal.h"

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c);      \
      ++fails;                                                     \
    }                                                              \
  } while (0)

int main() {
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<int64_t> xs) {
    auto it = xs.begin();
    std::advance(it, rng() % xs.size());
    return *it;
  };
  long planned = 0, rejected = 0;
  for (int it = 0; it < 200000; ++it) {
    rattn_problem p{};
    p.batch = (int32_t)pick({1, 2, 3, 16, 64, 255, 4096, 0, -1, 1 << 20});
    p.num_kv_heads = (int32_t)pick({1, 2, 8, 16, 0, 7});
    p.num_q_heads = p.num_kv_heads * (int32_t)pick({1, 4, 6, 8, 16, 64, 128}) +
                    (int32_t)pick({0, 0, 0, 0, 1});
    p.head_dim = (int32_t)pick({128, 128, 128, 64});
    p.n_query_rows = (int32_t)pick({1, 2, 3, 8, 9, 16, 21, 22, 33, 100, 2048, 0});
    p.page_size = (int32_t)pick({16, 32, 64, 256, 24, 8, 0, 1 << 20});
    p.max_seq_len = (int32_t)pick({1, 2, 31, 1000, 2048, 9000, 100000, 262144, 1048576,
                                   1 << 30, (1 << 30) + 1, 0, 2147483647});
    const int64_t ps = p.page_size > 0 ? p.page_size : 1;
    const int64_t need = (p.max_seq_len + ps - 1) / ps;
    p.max_pages_per_seq = (int32_t)std::min<int64_t>(need + pick({0, 0, 1, -1}), 2147483647);
    p.num_pages = (int32_t)pick({1, 100, 6251, 1 << 24, 2147483647});
    p.window = (int32_t)pick({0, 0, 1, 17, 512, 1024, 1 << 29, -1});
    p.dmax = (int32_t)pick({0, 3, 1024, 131071, 1048575, 2147483646, -1});
    p.softmax_scale = (float)pick({1, 1, 2}) * 0.08838834764831845f;
    p.kv_dtype = (int32_t)pick({0, 1, 2});
    p.num_splits = (int32_t)pick({0, 0, 0, 1, 2, 3, 7, 4096, 4097, -1});
    for (int32_t cus : {1, 80, 256, 304}) {
      rattn_plan_info info{};
      const rattn_status st = rattn_plan_describe(&p, cus, &info);
      if (st == RATTN_OK) {
        ++planned;
        // a grid's work-items stay below 2^31 (one work-group of row_tiles waves, or
        // pieces_per_group waves, each)
        CHECK(info.grid_x >= 1);
        CHECK((int64_t)info.grid_x * 64 * info.row_tiles * info.pieces_per_group <
              ((int64_t)1 << 31));
        if (info.kernel == RATTN_KERNEL_PREFILL) CHECK(info.combine_blocks == 0);
        CHECK(info.workspace_bytes >= 256);
        CHECK(info.row_tiles >= 1 && info.tiles_per_wave >= 1);
        CHECK(info.combine_blocks >= 0);
      } else {
        ++rejected;
        CHECK(st == RATTN_E_INVALID || st == RATTN_E_UNSUPPORTED);
      }
    }
    // host-side checks of the entry points, before any HIP call
    int32_t dummy = 0;
    const void* d = &dummy;
    CHECK(rattn_decode(nullptr, d, d, d, nullptr, nullptr, (const int32_t*)d,
                       (const int32_t*)d, (const float*)d, (void*)d, nullptr,
                       nullptr) == RATTN_E_INVALID);
    if (rattn::validate_problem(&p) != RATTN_OK) {
      CHECK(rattn_decode_static(&p, d, d, d, nullptr, nullptr, (const int32_t*)d,
                                (const int32_t*)d, (const float*)d, (void*)d, nullptr, nullptr,
                                nullptr) != RATTN_OK);
      CHECK(rattn_append_kv(&p, d, d, (const int32_t*)d, (const int32_t*)d, (void*)d, (void*)d,
                            nullptr, nullptr, nullptr, nullptr) != RATTN_OK);
    }
  }
  CHECK(rattn_plan_describe(nullptr, 256, nullptr) == RATTN_E_INVALID);
  CHECK(rattn_free(nullptr) == RATTN_OK);
  std::printf("%s %ld planned %ld rejected\n", fails ? "FAILED" : "ok", planned, rejected);
  return fails ? 1 : 0;
}
