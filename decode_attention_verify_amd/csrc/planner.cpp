// Problem validation and the split planner (host only, no HIP calls).
//
// The split count follows the idea on page 2 ("vLLM TML Inkling support", technical
// optimisation section, FA4 kernel): the key range is split, with the number of splits
// chosen from the batch size, the head count and the KV length. Here the planner picks
// the number of split work-groups from (batch * KV heads, visible KV span, compute
// units, resident work-groups per CU): the kernel divides the whole call's tiles evenly
// among them, so the choice sets occupancy. Pieces stay long where the round of
// resident work-groups is full (every piece of a shared unit costs a partial write and
// a combine read) and go down to one tile where the units are too few to fill it; units
// of two or three single-wave pieces are merged by one work-group with no combine.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "internal.h"

namespace rattn {

static bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Tiles of one (sequence, KV head) unit at the planning length: the keys visible to at
// least one row, plus the slack of aligning the first key down to a tile boundary.
static int64_t unit_tiles_bound(const rattn_problem& p) {
  int64_t span = p.window > 0
                     ? std::min<int64_t>(p.max_seq_len, (int64_t)p.window + p.n_query_rows - 1)
                     : p.max_seq_len;
  span += kTileKeys - 1;
  return (span + kTileKeys - 1) / kTileKeys;
}

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
  // a positive normal float: the kernels divide the bias by it and take maxima of s / scale
  if (!std::isnormal(p->softmax_scale) || !(p->softmax_scale > 0.f)) return RATTN_E_INVALID;
  if (p->kv_dtype != RATTN_KV_BF16 && p->kv_dtype != RATTN_KV_FP8_E4M3) return RATTN_E_INVALID;
  if (p->num_splits < 0) return RATTN_E_INVALID;
  // valid, but outside what the kernels implement
  if (p->head_dim != kHeadDim) return RATTN_E_UNSUPPORTED;
  const int32_t G = p->num_q_heads / p->num_kv_heads;
  const int64_t rows = (int64_t)G * p->n_query_rows;
  if (rows > kMaxRows) {
    // many rows per sequence: the prefill kernel, for the group sizes it is built for,
    // without forced splits
    if (prefill_heads_per_wave(G) == 0) return RATTN_E_UNSUPPORTED;
    if (p->num_splits != 0) return RATTN_E_UNSUPPORTED;
    // one 8-wave work-group per (sequence, KV head, block of query tokens): the grid's
    // work-items must stay below 2^31
    const int64_t blocks = (p->n_query_rows + prefill_tokens(G) - 1) / prefill_tokens(G);
    if (((int64_t)p->batch * p->num_kv_heads * blocks + 7) * 64 * kPrefillWaves >=
        ((int64_t)1 << 31))
      return RATTN_E_UNSUPPORTED;
  } else if (split_shape(*p).waves == 0) {
    // a tile's bias slice (G heads x (32 + n - 1) distances) must fit the work-group's
    // loads
    return RATTN_E_UNSUPPORTED;
  }
  if (!is_pow2(p->page_size) || p->page_size < 16) return RATTN_E_UNSUPPORTED;
  if (p->max_seq_len > (1 << 30)) return RATTN_E_UNSUPPORTED;
  if (p->num_splits > kMaxSplits) return RATTN_E_UNSUPPORTED;
  // the bias table is indexed with 32-bit element offsets
  if ((int64_t)p->num_q_heads * ((int64_t)p->dmax + 1) > INT32_MAX) return RATTN_E_UNSUPPORTED;
  // the split kernel counts the call's tiles (every unit's, at lengths up to
  // max_seq_len) in 32-bit integers: their sum must stay below 2^31
  const int64_t total = (int64_t)p->batch * p->num_kv_heads * unit_tiles_bound(*p);
  if (total > INT32_MAX) return RATTN_E_UNSUPPORTED;
  // a split grid holds at least one work-group of up to 8 waves per (sequence, KV head)
  // unit; its work-items must stay below 2^31
  if (rows <= kMaxRows &&
      (int64_t)p->batch * p->num_kv_heads * 64 * kMaxWaves >= ((int64_t)1 << 31))
    return RATTN_E_UNSUPPORTED;
  return RATTN_OK;
}

bool uses_even_shares(const rattn_problem& p) {
  // full-context layers over a batch: sequence lengths may differ by a large factor
  return p.num_splits == 0 && p.window == 0 && p.batch > 1;
}

// Chunked prefill: one work-group per (sequence, KV head, block of query tokens), each
// over all the keys its rows see; the grid is rounded up to a multiple of the 8 XCDs
// (the kernel numbers its work-groups per XCD). No partials, no combine.
static Plan make_prefill_plan(const rattn_problem& p, int32_t num_cus, int32_t blocks_per_cu) {
  const int32_t G = p.num_q_heads / p.num_kv_heads;
  Plan pl{};
  pl.prefill = 1;
  pl.prefill_hw = prefill_heads_per_wave(G);
  pl.ws = 1;
  pl.rt = 1;
  pl.waves = kPrefillWaves;
  pl.num_cus = num_cus;
  pl.blocks_per_cu = blocks_per_cu;
  const int64_t blocks = (p.n_query_rows + prefill_tokens(G) - 1) / prefill_tokens(G);
  const int64_t groups = (int64_t)p.batch * p.num_kv_heads * blocks;
  pl.split_groups = (int32_t)((groups + 7) / 8 * 8);
  pl.splits_per_unit = 1;
  pl.num_splits = 1;
  pl.keys_per_split = p.max_seq_len;
  pl.workspace_bytes = 256;                  // the flag word only
  return pl;
}

Plan make_plan(const rattn_problem& p, int32_t num_cus, int32_t blocks_per_cu) {
  const int32_t G = p.num_q_heads / p.num_kv_heads;
  const int32_t rows = G * p.n_query_rows;
  if (rows > kMaxRows) return make_prefill_plan(p, num_cus, blocks_per_cu);
  Plan pl{};
  const SplitShape sh = split_shape(p);
  pl.rt = sh.rt;
  pl.waves = sh.waves;
  pl.num_cus = num_cus;
  pl.blocks_per_cu = blocks_per_cu;
  const int64_t units = (int64_t)p.batch * p.num_kv_heads;
  const int64_t tiles = unit_tiles_bound(p);
  const int64_t total = units * tiles;       // tiles of the whole call at the bound
  // The grid is one round of resident work-groups. Single-wave groups over a bf16
  // cache fill three quarters of it: on MI355X a 100K-key batch-1 decode streams
  // fastest with 3 of the 4 resident single-wave groups per CU busy (6.26 TB/s, against
  // 6.16 at 4 and 6.06 at 2), and an integral count per CU beats a fractional one.
  // Groups whose per-tile work, not HBM, bounds them fill the whole round: multi-wave
  // groups (the 8-row verify workload: 2.57 ms at a full round against 3.30 ms at three
  // quarters) and the E4M3 cache, which decodes every element (the 1M-key decode:
  // 529 us against 542 us).
  // Per-unit splits go down to one tile per piece when the units are too few to fill the
  // round otherwise: the pieces of a latency-bound call end sooner than fewer, longer
  // ones, partial and merge included (2K-key decode on 6q/1kv: 64 one-tile pieces
  // 11.0 us, 16 pieces of 4 tiles 13.5; the window layer at batch 1, 8 units: 32 pieces
  // per unit 12.8 us, 8 pieces 15.7). Even shares keep at least 4 tiles per work-group.
  // Units of multi-wave groups stay whole when they alone give
  // every CU four waves: then splitting buys little and the merge of their many rows
  // costs more (9-row verify over W = 512 on 64q/16kv, 256 units: 26.6 us whole against
  // 30.7 us in two pieces, 7 us of it the merge; the 8-row verify over W = 1024 on
  // 48q/8kv has 128 units and is fastest in four pieces, 30.2 us against 32.3 in two).
  const int64_t slots = (int64_t)std::max(num_cus, 1) * std::max(blocks_per_cu, 1);
  const bool latency_bound = pl.waves > 1 || pl.rt > 1 || p.kv_dtype == RATTN_KV_FP8_E4M3;
  const int64_t target = std::max<int64_t>(1, latency_bound ? slots : slots * 3 / 4);
  int64_t k = 0;                             // pieces per unit; 0 = even shares
  int64_t groups;
  if (p.num_splits > 0) {
    k = std::min<int64_t>(p.num_splits, std::max<int64_t>(1, kMaxGroups / units));
    groups = k * units;
  } else if (!uses_even_shares(p)) {
    // every unit spans about the same keys (a window, or a single sequence): an equal
    // number of pieces per unit is balanced and needs no search for a work-group's unit
    k = std::max<int64_t>(1, std::min<int64_t>(target / units, tiles));
    if (pl.waves * pl.rt > 1 &&
        units * pl.waves * pl.rt >= 4 * (int64_t)std::max(num_cus, 1))
      k = 1;
    k = std::min<int64_t>(k, std::max<int64_t>(1, kMaxGroups / units));
    groups = k * units;
  } else {
    // full-context layers over a batch: lengths may differ by a large factor, so the
    // whole call's tiles are shared evenly
    groups = std::min<int64_t>(target, std::max<int64_t>(1, total / 4));
    groups = std::max<int64_t>(1, std::min<int64_t>(groups, kMaxGroups));
  }
  // Units of single-wave bf16 pieces that would get at most kMergeWaves pieces each run
  // as one work-group of w waves per unit, w pieces merged by the group itself, with no
  // partials and no combine: w = 3 where a group fits on every unit's own CU (units <=
  // CUs), w = 2 where two groups share a CU (units <= 2 CUs), pieces of 4 tiles or more.
  // On MI355X: the 64q/16kv window layer at batch 16 (256 units, 3 merged pieces)
  // 15.9 us against 19.5 with three single-wave groups and the combine; the 48q/8kv
  // window layer at batch 64 (512 units) 45.4-45.8 us in 2 merged pieces against
  // 49-51 whole (two waves per CU) and 51.7 in 2 pieces with the combine. At 6 pieces
  // per unit the combine stays faster (48q/8kv window layer, batch 16: 19.6 us against
  // 20.6-21.0 at 3 merged). A forced split of 2 or 3 pieces merges the same way.
  pl.ws = 1;
  if (pl.waves == 1 && pl.rt == 1 && p.kv_dtype == RATTN_KV_BF16 && k >= 1) {   // per-unit
    int64_t w = 1;
    if (p.num_splits > 0) {
      w = (k == 2 || k == kMergeWaves) ? k : 1;
    } else if (k <= kMergeWaves) {
      const int64_t cus = std::max(num_cus, 1);
      if (units <= cus && tiles / 4 >= 3) w = 3;
      else if (units <= 2 * cus && tiles / 4 >= 2) w = 2;
    }
    if (w > 1) {
      k = w;
      pl.ws = (int32_t)w;
      groups = units;
    }
  }
  pl.split_groups = (int32_t)groups;
  pl.splits_per_unit = (int32_t)k;
  pl.num_splits = (int32_t)(k > 0 ? k : (groups + units - 1) / units);
  const int64_t npieces = groups * pl.ws;
  pl.keys_per_split = (int32_t)std::min<int64_t>(((total + npieces - 1) / npieces) * kTileKeys,
                                                 INT32_MAX);
  int64_t pieces = 0;                        // partial slots
  if (k > 1 && pl.ws == 1) pieces = groups;
  if (k == 0 && groups > 1) pieces = groups + units;
  pl.part_o_floats = pieces * rows * kHeadDim;
  pl.part_lse_floats = pieces * rows;
  pl.unit_info_ints = k == 0 ? 2 * units : 0;
  // partials, unit records, then a 256-byte aligned flag word
  int64_t bytes = (pl.part_o_floats + pl.part_lse_floats + pl.unit_info_ints) * 4;
  bytes = (bytes + 255) / 256 * 256;
  pl.workspace_bytes = bytes + 256;
  return pl;
}

// The combine's shape for a partition (see combine_kernel), with what chose it on MI355X:
//  * per-unit splits of up to 16 pieces: whole rows, 2 stripes of 32 lanes, 4 rows per
//    work-group, 8 pieces in flight per thread (the window layer at batch 16, 6 pieces
//    per unit: 18.2 us per call against 19.3 with 1 stripe and 8 rows per work-group);
//  * even shares (a few to a few tens of pieces per unit): the same, 16 pieces in flight;
//  * 17 to 255 pieces: one wave per 16-dim slice of a row, 16 stripes of 4 lanes (the
//    100K-key decode's 96 pieces merge 0.4 us sooner than in 32-dim slices of 8 stripes,
//    65 pieces 0.7 us sooner; 32 stripes per 8-dim slice were no faster, 64 per 4-dim
//    slice slower);
//  * 256 pieces or more: 16 waves per 32-dim slice, 128 stripes of 8 lanes; for a call of
//    fewer than 32 rows, per 16-dim slice, 256 stripes of 4 lanes, so that the few rows
//    spread over twice the work-groups (one rank's share of the 100K-key layer under
//    8-way tensor parallelism, 6 rows of 768 pieces: 0.4 us sooner, under 4-way 0.7 us;
//    the 1M-key E4M3 decode, 48 rows of 256 pieces, merged 1.2 us later that way).
CombineShape combine_shape(int64_t rows, int splits_per_unit) {
  if (splits_per_unit == 0) return kCombineRows2;
  if (splits_per_unit <= 16) return kCombineRows;
  if (splits_per_unit >= 256) return rows < 32 ? kCombineWide16 : kCombineWide;
  return kCombineSlices;
}

int64_t combine_blocks(int64_t rows, int splits_per_unit) {
  switch (combine_shape(rows, splits_per_unit)) {
    case kCombineRows:
    case kCombineRows2: return (rows + 3) / 4;
    case kCombineWide: return rows * 4;   // one work-group per 32-dim slice of a row
    default: return rows * 8;             // one work-group per 16-dim slice of a row
  }
}

}  // namespace rattn
