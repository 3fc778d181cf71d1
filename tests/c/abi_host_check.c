/* The C ABI from plain C on the host (no GPU call): the header compiles as C, the library
 * links, host-side validation and the planner answer, and status strings are defined.
 * Built and run by tests/test_c_abi.py; prints one line per check and exits non-zero on
 * the first failure. */
#include <stdio.h>
#include <string.h>

#include "rattn.h"

static int fails = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++fails;
}

static rattn_problem headline(void) {
  rattn_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.num_q_heads = 48;
  p.num_kv_heads = 8;
  p.head_dim = 128;
  p.n_query_rows = 1;
  p.page_size = 16;
  p.num_pages = 6251;
  p.max_pages_per_seq = 6250;
  p.max_seq_len = 100000;
  p.window = 0;
  p.dmax = 131071;
  p.softmax_scale = 0.08838834764831845f;
  p.kv_dtype = RATTN_KV_BF16;
  p.num_splits = 0;
  return p;
}

int main(void) {
  rattn_plan_info info;
  rattn_problem p = headline();
  check(rattn_abi_version() == RATTN_ABI_VERSION, "ABI version matches the header");
  check(rattn_plan_describe(&p, 256, &info) == RATTN_OK, "headline plans");
  check(info.kernel == RATTN_KERNEL_SPLIT_KV && info.grid_x > 0 && info.row_tiles == 1,
        "headline uses the split kernel with single-wave pieces");
  check(info.pieces_per_group == 1 && info.combine_blocks > 0,
        "headline splits its units and merges them in the combine");
  check((int64_t)info.grid_x * info.pieces_per_group * info.keys_per_split >=
            (int64_t)8 * 100000,
        "the split covers every key of every KV head");
  p = headline();
  p.num_splits = 3;
  check(rattn_plan_describe(&p, 256, &info) == RATTN_OK && info.pieces_per_group == 3 &&
            info.combine_blocks == 0 && info.grid_x == 8,
        "three pieces per unit: one work-group per unit merges them");
  p = headline();
  p.n_query_rows = 2048;
  check(rattn_plan_describe(&p, 256, &info) == RATTN_OK && info.kernel == RATTN_KERNEL_PREFILL &&
            info.combine_blocks == 0,
        "a 2048-row chunk plans the prefill kernel");
  p = headline();
  p.batch = 0;
  check(rattn_plan_describe(&p, 256, &info) == RATTN_E_INVALID, "batch 0 is invalid");
  p = headline();
  p.head_dim = 64;
  check(rattn_plan_describe(&p, 256, &info) == RATTN_E_UNSUPPORTED, "head_dim 64 is unsupported");
  check(rattn_plan_describe(NULL, 256, &info) == RATTN_E_INVALID, "a null problem is invalid");
  check(rattn_free(NULL) == RATTN_OK, "freeing a null plan is a no-op");
  check(rattn_decode(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) ==
            RATTN_E_INVALID,
        "a decode without a plan is invalid");
  check(strlen(rattn_status_string(RATTN_E_HIP)) > 0, "status strings are defined");
  return fails != 0;
}
