// Internal declarations shared by the host library (api.cpp, planner.cpp) and the
// kernels (kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/rattn.h"

namespace rattn {

constexpr int kHeadDim = 128;     // head size of every layer (page 2, model architecture)
constexpr int kTileKeys = 32;     // keys per inner-loop step: two 16-key MFMA subtiles
constexpr int kMaxRows = 64;      // packed query rows per (sequence, KV head): 4 row tiles
constexpr int kMaxSplits = 4096;
constexpr int kChunkPages = 512;   // page ids staged in LDS per chunk of a split
constexpr int kCombineSlices = 4;   // combine work-groups per output row (32 dims each)

// Planner output: how one rattn_decode call is launched.
struct Plan {
  int32_t num_splits;
  int32_t keys_per_split;
  int32_t row_tiles;
  int32_t num_cus;
  int32_t blocks_per_cu;
  int64_t workspace_bytes;
  int64_t part_o_floats;    // [batch][n][Hq][splits][D]
  int64_t part_lse_floats;  // [batch][n][Hq][splits]
};

// Host-side validation of a problem; no HIP call.
rattn_status validate_problem(const rattn_problem* p);

// Split-kernel work-groups that stay resident on one CU at a time, as measured for
// the gfx950 build (one wave per SIMD); rattn_plan queries the runtime instead.
constexpr int kDefaultBlocksPerCU = 4;

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
  int32_t* flags;
  int32_t batch, n, num_q_heads, num_kv_heads, group;   // group = Hq / Hkv
  int32_t page_size, page_shift, num_pages, max_pages;
  int32_t max_seq_len, window, dmax;
  float softmax_scale;
  int32_t num_splits, keys_per_split;
};

// Kernel launchers (kernels.hip). Return 0 on success, else a hipError_t value.
int launch_split_kv(const KernelArgs& a, int row_tiles, bool fp8, void* stream);
int launch_combine(const KernelArgs& a, void* stream);
// Resident split-kernel work-groups per CU for this variant (0 if the query fails).
int split_kv_blocks_per_cu(int row_tiles, bool fp8);

}  // namespace rattn
