// Problem validation and the split planner (host only, no HIP calls).
//
// The split count follows the idea on page 2 ("vLLM TML Inkling support", technical
// optimisation section, FA4 kernel): the number of key-range splits is chosen from the
// batch size, the head count and the KV length. Here the key is
// (batch * KV heads, packed rows, visible KV span, compute units): enough work-groups
// to fill every CU several times over, but no split shorter than a few tiles, because
// every split costs a partial write and a combine read.
#include <cmath>

#include "internal.h"

namespace rattn {

static bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

rattn_status validate_problem(const rattn_problem* p) {
  if (p == nullptr) return RATTN_E_INVALID;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1) return RATTN_E_INVALID;
  if (p->num_q_heads % p->num_kv_heads != 0) return RATTN_E_INVALID;
  if (p->n_query_rows < 1) return RATTN_E_INVALID;
  if (p->page_size < 1 || p->num_pages < 1 || p->max_pages_per_seq < 1) return RATTN_E_INVALID;
  if (p->max_seq_len < p->n_query_rows) return RATTN_E_INVALID;
  if ((int64_t)p->max_seq_len > (int64_t)p->max_pages_per_seq * p->page_size)
    return RATTN_E_INVALID;
  if (p->window < 0 || p->dmax < 0) return RATTN_E_INVALID;
  if (!std::isfinite(p->softmax_scale)) return RATTN_E_INVALID;
  if (p->kv_dtype != RATTN_KV_BF16 && p->kv_dtype != RATTN_KV_FP8_E4M3) return RATTN_E_INVALID;
  if (p->num_splits < 0) return RATTN_E_INVALID;
  // valid, but outside what the kernels implement
  if (p->head_dim != kHeadDim) return RATTN_E_UNSUPPORTED;
  const int64_t rows = (int64_t)(p->num_q_heads / p->num_kv_heads) * p->n_query_rows;
  if (rows > kMaxRows) return RATTN_E_UNSUPPORTED;
  if (!is_pow2(p->page_size) || p->page_size < 16) return RATTN_E_UNSUPPORTED;
  if (p->max_seq_len > (1 << 30)) return RATTN_E_UNSUPPORTED;
  if (p->num_splits > kMaxSplits) return RATTN_E_UNSUPPORTED;
  return RATTN_OK;
}

Plan make_plan(const rattn_problem& p, int32_t num_cus, int32_t blocks_per_cu) {
  const int32_t G = p.num_q_heads / p.num_kv_heads;
  const int32_t rows = G * p.n_query_rows;
  Plan pl{};
  pl.row_tiles = (rows + 15) / 16;
  pl.num_cus = num_cus;
  pl.blocks_per_cu = blocks_per_cu;
  // keys visible to at least one row, plus the slack of aligning the first key down
  // to a tile boundary
  int64_t span = p.window > 0 ? std::min<int64_t>(p.max_seq_len, (int64_t)p.window +
                                                  p.n_query_rows - 1)
                              : p.max_seq_len;
  span += kTileKeys - 1;
  const int64_t tiles = (span + kTileKeys - 1) / kTileKeys;
  int64_t splits;
  if (p.num_splits > 0) {
    splits = p.num_splits;
  } else {
    // One single-wave work-group per split. The grid is sized to one round of resident
    // work-groups, filled to three quarters: on MI355X a 100K-key batch-1 decode streams
    // fastest with 3 of the 4 resident waves per CU busy (6.26 TB/s, against 6.16 at 4
    // and 6.06 at 2), and one round avoids a partly idle second round.
    const int64_t units = (int64_t)p.batch * p.num_kv_heads;
    const int64_t slots = (int64_t)std::max(num_cus, 1) * std::max(blocks_per_cu, 1);
    const int64_t target = std::max<int64_t>(1, slots * 3 / 4);
    splits = (target + units - 1) / units;
    const int64_t min_tiles = 4;   // at least 128 keys per split
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, tiles / min_tiles));
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, kMaxSplits));
  }
  const int64_t tiles_per_split = (tiles + splits - 1) / splits;
  if (p.num_splits == 0) splits = (tiles + tiles_per_split - 1) / tiles_per_split;
  pl.num_splits = (int32_t)splits;
  pl.keys_per_split = (int32_t)(tiles_per_split * kTileKeys);
  if (pl.num_splits > 1) {
    const int64_t rows_total = (int64_t)p.batch * p.n_query_rows * p.num_q_heads;
    pl.part_o_floats = rows_total * pl.num_splits * kHeadDim;
    pl.part_lse_floats = rows_total * pl.num_splits;
  }
  // partials, then a 256-byte aligned flag word
  int64_t bytes = (pl.part_o_floats + pl.part_lse_floats) * 4;
  bytes = (bytes + 255) / 256 * 256;
  pl.workspace_bytes = bytes + 256;
  return pl;
}

}  // namespace rattn
