// Internal declarations shared by the host library (api.cpp, planner.cpp) and the
// kernels (kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/rattn.h"

namespace rattn {

constexpr int kHeadDim = 128;     // head size of every layer (page 2, model architecture)
constexpr int kTileKeys = 32;     // keys per inner-loop step: two 16-key MFMA subtiles
constexpr int kMaxRows = 128;     // packed query rows per (sequence, KV head): 8 waves
constexpr int kMaxSplits = 4096;  // largest forced split count per (sequence, KV head)
constexpr int kMaxGroups = 1 << 16;   // largest split-kernel grid
constexpr int kChunkPages = 512;  // page ids staged in LDS per chunk of a piece

// Bias slice of one tile: G heads x (32 + n - 1) distances, loaded by the work-group's
// threads with kBiasPerThread loads each.
constexpr int kBiasPerThread = 4;
constexpr int kMaxWaves = 8;      // waves of a split work-group (one 16-row tile each)
// A one-wave piece of several row tiles loads the slice alone: 8 loads per lane
constexpr int kBiasPerThreadRows = 8;
// Four waves of two row tiles: 2 loads per lane (slices of up to 512 entries: the 9-row
// step of an 8-head group needs 320), which keeps the two tiles in flight in registers
constexpr int kBiasPerThreadPair = 2;
constexpr int kMaxRowTiles = 3;   // row tiles of a one-wave piece (48 rows)

// Waves per split work-group for G query heads per KV head and n rows: each wave owns
// one 16-row MFMA tile of ceil(G n / waves) rows (1, 2, 4 or 8 waves for up to 16, 32,
// 64 or 128 rows; 8 waves run two per SIMD, one work-group per CU). A multi-wave
// group's threads must cover a tile's bias slice with kBiasPerThread loads each (a
// single wave gathers its own). Returns 0 when 8 waves do not suffice.
inline int waves_for(int G, int n) {
  const int rows = G * n;
  if (rows > kMaxRows) return 0;
  if (rows <= 16) return 1;
  int w = rows <= 32 ? 2 : (rows <= 64 ? 4 : 8);
  const int slice = G * (kTileKeys + n - 1);
  while (w < kMaxWaves && slice > 64 * w * kBiasPerThread) w *= 2;
  return slice <= 64 * w * kBiasPerThread ? w : 0;
}

// Row tiles per wave. Over a bf16 cache whose rows all see at least kRowTilesMinSpan
// keys, a piece of 17 to 48 packed rows runs as one wave of 2 or 3 row tiles (16 rows
// each, or fewer rows spread evenly over them), and a piece of 65 to 128 rows whose bias
// slice has at most 512 entries as four waves of two row tiles (up to 32 rows per wave);
// other row counts, slices and spans keep one row tile per wave (waves_for). A wave reads each K and V fragment once for its tiles.
// On MI355X the 8-row verify of 6-head groups over 32K-256K keys ran 7 % faster as one
// wave of three tiles than as four waves of one, the same step over a 1,024-key window
// 26 % slower. (4 and 5 tiles per wave spill registers.)
constexpr int kRowTilesMinSpan = 8192;

struct SplitShape {
  int waves;   // waves per split work-group (0: none fits)
  int rt;      // row tiles per wave
};

// The split kernel's layout for a problem of at most kMaxRows packed rows per unit.
inline SplitShape split_shape(const rattn_problem& p) {
  const int G = p.num_q_heads / p.num_kv_heads;
  const int n = p.n_query_rows;
  const int64_t rows = (int64_t)G * n;
  const int64_t span = p.window > 0 ? (int64_t)p.window : (int64_t)p.max_seq_len;
  const int64_t slice = (int64_t)G * (kTileKeys + n - 1);
  if (p.kv_dtype == RATTN_KV_BF16 && span >= kRowTilesMinSpan) {
    if (rows > 16 && rows <= 16 * kMaxRowTiles && slice <= 64 * kBiasPerThreadRows)
      return SplitShape{1, (int)((rows + 15) / 16)};
    if (rows > 64 && rows <= kMaxRows && slice <= 64 * 4 * kBiasPerThreadPair)
      return SplitShape{4, 2};
  }
  return SplitShape{waves_for(G, n), 1};
}

// A unit of single-wave bf16 pieces split in 2 or kMergeWaves pieces runs as one
// work-group of that many waves, one piece each, which merges them into the unit's
// output, so that no combine launch follows (a wave per SIMD: one 3-wave group or two
// 2-wave groups per CU).
constexpr int kMergeWaves = 3;

// Chunked prefill (G n > kMaxRows): heads per wave of the prefill kernel for G query
// heads per KV head, 0 if not built. Each head costs a wave 48 registers (its 16 rows'
// O accumulators and queries): 3 heads of a 6-head group and 2 of a 4- or 8-head group
// fit the 256 registers of a wave that shares its SIMD with a second one.
inline int prefill_heads_per_wave(int G) {
  return G == 6 ? 3 : ((G == 4 || G == 8) ? 2 : 0);
}
// Waves per prefill work-group: 8, two per SIMD, so that one wave's exponentials overlap
// the other's matrix instructions (with 4 waves, one per SIMD, the same kernel ran at
// 410-520 TFLOP/s against 710-800 with 8).
constexpr int kPrefillWaves = 8;
// Query tokens per prefill work-group: its waves cover kPrefillWaves / (G / heads per
// wave) blocks of 16 tokens (64 tokens for 4- and 6-head groups, 32 for 8-head groups).
inline int prefill_tokens(int G) {
  const int hw = prefill_heads_per_wave(G);
  return hw ? 16 * (kPrefillWaves / (G / hw)) : 0;
}

// Planner output: how one rattn_decode call is launched.
struct Plan {
  int32_t split_groups;     // split-kernel work-groups (the grid)
  int32_t waves;            // waves per split work-group
  int32_t num_splits;       // nominal work-groups per (sequence, KV head) unit
  int32_t keys_per_split;   // nominal keys per work-group at the planning length
  int32_t num_cus;
  int32_t blocks_per_cu;
  int64_t workspace_bytes;
  int32_t splits_per_unit;  // > 0: per-unit split into this many pieces; 0: even shares
  int64_t part_o_floats;    // [pieces][rows per unit][D]
  int64_t part_lse_floats;  // [pieces][rows per unit]
  int64_t unit_info_ints;   // even shares: [units][2] (first work-group, pieces)
  int32_t prefill;          // 1: the prefill kernel (many rows per sequence), no combine
  int32_t prefill_hw;       // heads per wave of the prefill kernel
  int32_t ws;               // pieces per split work-group (2 or 3: merged in it)
  int32_t rt;               // 16-row tiles per wave (> 1: one wave holds all the rows)
};

// Host-side validation of a problem; no HIP call.
rattn_status validate_problem(const rattn_problem* p);

// Split-kernel work-groups that stay resident on one CU at a time, as measured for
// the gfx950 build (one wave per SIMD); rattn_plan queries the runtime instead.
constexpr int kDefaultBlocksPerCU = 4;

// Whether the planner shares the whole call's tiles evenly among the work-groups (else
// it splits every (sequence, KV head) unit into the same number of pieces).
bool uses_even_shares(const rattn_problem& p);

// Host-side planner; no HIP call. `p` must be valid.
Plan make_plan(const rattn_problem& p, int32_t num_cus, int32_t blocks_per_cu);

// Arguments of the split-KV kernel and of the combine kernel.
struct KernelArgs {
  const uint16_t* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const float* bias;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int32_t* unit_info;
  int32_t* flags;
  // rows per sequence: null = n rows each, sequence b at rows b*n ..; else sequence b
  // owns packed rows cu_rows[b] .. cu_rows[b+1]-1 (at most n) of row_cap rows
  const int32_t* cu_rows;
  int32_t row_cap;
  int32_t batch, n, num_q_heads, num_kv_heads, group;   // group = Hq / Hkv
  int32_t page_size, page_shift, num_pages, max_pages;
  int32_t max_seq_len, window, dmax;
  float softmax_scale;
  int32_t split_groups;     // grid of the split kernel
  int32_t splits_per_unit;  // > 0: pieces per unit; 0: even shares of all tiles
};

// Arguments of the KV-cache append kernel.
struct AppendArgs {
  const uint16_t* k_new;    // bf16 [batch][n][Hkv][D]
  const uint16_t* v_new;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* k_cache;            // bf16 or E4M3 codes [num_pages][Hkv][page_size][D]
  void* v_cache;
  float* k_scale;           // fp32 [num_pages][Hkv][page_size] (E4M3 only)
  float* v_scale;
  int32_t* flags;           // RATTN_FLAG_* bits, or null
  int32_t batch, n, num_kv_heads, page_size, page_shift, num_pages, max_pages, max_seq_len;
  int32_t fp8;
};

constexpr float kE4M3Max = 448.f;

// Kernel launchers (kernels.hip). Return 0 on success, else a hipError_t value. With a
// pair of events (hipEvent_t), the launch stamps them with the kernel's start and end.
int launch_split_kv(const KernelArgs& a, int waves, bool fp8, int ws, int rt, void* stream,
                    void* ev_start = nullptr, void* ev_stop = nullptr);
int launch_combine(const KernelArgs& a, void* stream, void* ev_start = nullptr,
                   void* ev_stop = nullptr);
// The combine kernel's shape for `rows` output rows and the partition (planner.cpp),
// and its work-groups (host functions).
enum CombineShape { kCombineRows, kCombineRows2, kCombineSlices, kCombineWide, kCombineWide16 };
CombineShape combine_shape(int64_t rows, int splits_per_unit);
int64_t combine_blocks(int64_t rows, int splits_per_unit);
int launch_append_kv(const AppendArgs& a, void* stream);

// The static scratch array of rattn_decode_static (scratch.hip): its size, and its
// address on `device`, which must be the current device on the first call for that
// device (resolved then with hipGetSymbolAddress and kept). Returns 0 or a hipError_t.
constexpr int64_t kStaticScratchBytes = (int64_t)32 << 20;
int static_scratch_ptr(int device, void** ptr);
int launch_prefill(const KernelArgs& a, int heads_per_wave, int group, bool fp8, void* stream,
                   void* ev_start = nullptr, void* ev_stop = nullptr);
int launch_read_probe(const void* buf, int64_t nblocks, int block_bytes, const int32_t* order,
                      int waves, void* sink, void* stream);
// Resident split-kernel work-groups per CU for this variant (0 if the query fails).
int split_kv_blocks_per_cu(int waves, bool fp8, bool even, int rt);

}  // namespace rattn
