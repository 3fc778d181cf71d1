// C ABI of librattn: plan, decode, free, plus instrumentation. Host code.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "internal.h"

struct rattn_plan_s {
  rattn_problem prob;
  rattn::Plan plan;
  int device;
  void* workspace;          // partials, then the flag word
  int32_t* flags;
  // instrumentation
  int32_t prof_max;
  int32_t prof_count;
  int32_t prof_stride;      // record every prof_stride-th call
  int64_t prof_calls;       // calls since rattn_profile_begin
  std::vector<hipEvent_t> prof_events;   // 4 per call: split start/end, combine start/end
};

namespace {

bool log_enabled() {
  const char* e = std::getenv("RATTN_LOG");
  return e != nullptr && e[0] != '\0' && e[0] != '0';
}

// Some unit is shared by several work-groups, so a combine launch merges partials.
bool needs_combine(const rattn::Plan& pl) {
  if (pl.ws > 1) return false;               // merged by the split kernel itself
  return pl.splits_per_unit > 1 || (pl.splits_per_unit == 0 && pl.split_groups > 1);
}

void fill_info(const rattn_problem& p, const rattn::Plan& pl, rattn_plan_info* info) {
  info->num_splits = pl.num_splits;
  info->keys_per_split = pl.keys_per_split;
  info->tile_keys = rattn::kTileKeys;
  info->row_tiles = pl.waves;
  info->grid_x = pl.split_groups;
  info->grid_y = 1;
  info->grid_z = 1;
  info->combine_blocks =
      needs_combine(pl) ? (int32_t)rattn::combine_blocks(
                              (int64_t)p.batch * p.n_query_rows * p.num_q_heads,
                              pl.splits_per_unit)
                        : 0;
  info->num_cus = pl.num_cus;
  info->blocks_per_cu = pl.blocks_per_cu;
  info->kernel = pl.prefill ? RATTN_KERNEL_PREFILL : RATTN_KERNEL_SPLIT_KV;
  info->pieces_per_group = pl.prefill ? 1 : pl.ws;
  info->workspace_bytes = pl.workspace_bytes;
  info->tiles_per_wave = pl.prefill ? 1 : pl.rt;
}

void destroy_events(rattn_plan_s* p) {
  for (hipEvent_t e : p->prof_events) (void)hipEventDestroy(e);
  p->prof_events.clear();
  p->prof_max = 0;
  p->prof_count = 0;
  p->prof_stride = 1;
  p->prof_calls = 0;
}

}  // namespace

extern "C" {

int32_t rattn_abi_version(void) { return RATTN_ABI_VERSION; }

const char* rattn_status_string(rattn_status s) {
  switch (s) {
    case RATTN_OK: return "ok";
    case RATTN_E_INVALID: return "invalid argument";
    case RATTN_E_UNSUPPORTED: return "unsupported problem";
    case RATTN_E_HIP: return "HIP error";
    case RATTN_E_NOMEM: return "out of device memory";
  }
  return "unknown status";
}

rattn_status rattn_plan_describe(const rattn_problem* prob, int32_t num_cus,
                                 rattn_plan_info* info) {
  if (info == nullptr || num_cus < 1) return RATTN_E_INVALID;
  rattn_status st = rattn::validate_problem(prob);
  if (st != RATTN_OK) return st;
  fill_info(*prob, rattn::make_plan(*prob, num_cus, rattn::kDefaultBlocksPerCU), info);
  return RATTN_OK;
}

rattn_status rattn_plan(const rattn_problem* prob, rattn_plan_t* plan_out) {
  if (plan_out == nullptr) return RATTN_E_INVALID;
  *plan_out = nullptr;
  rattn_status st = rattn::validate_problem(prob);
  if (st != RATTN_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RATTN_E_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return RATTN_E_HIP;
  rattn_plan_s* p = new (std::nothrow) rattn_plan_s();
  if (p == nullptr) return RATTN_E_NOMEM;
  p->prob = *prob;
  const int G = prob->num_q_heads / prob->num_kv_heads;
  const rattn::SplitShape sh = rattn::split_shape(*prob);
  int bpc = (int64_t)G * prob->n_query_rows > rattn::kMaxRows
                ? 1
                : rattn::split_kv_blocks_per_cu(sh.waves, prob->kv_dtype == RATTN_KV_FP8_E4M3,
                                                rattn::uses_even_shares(*prob), sh.rt);
  if (bpc < 1) bpc = rattn::kDefaultBlocksPerCU;
  p->plan = rattn::make_plan(*prob, cus, bpc);
  p->device = dev;
  if (hipMalloc(&p->workspace, (size_t)p->plan.workspace_bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete p;
    return RATTN_E_NOMEM;
  }
  p->flags = (int32_t*)((char*)p->workspace + p->plan.workspace_bytes - 256);
  if (hipMemset(p->flags, 0, 256) != hipSuccess) {
    (void)hipFree(p->workspace);
    delete p;
    return RATTN_E_HIP;
  }
  if (log_enabled()) {
    std::fprintf(stderr,
                 "[rattn] plan: batch=%d n=%d Hq=%d Hkv=%d W=%d max_seq_len=%d kv=%s CUs=%d -> "
                 "groups=%d (%d per unit, %d keys each) waves=%d blocks/CU=%d "
                 "workspace=%lld B\n",
                 prob->batch, prob->n_query_rows, prob->num_q_heads, prob->num_kv_heads,
                 prob->window, prob->max_seq_len, prob->kv_dtype ? "e4m3" : "bf16", cus,
                 p->plan.split_groups, p->plan.num_splits, p->plan.keys_per_split,
                 p->plan.waves, p->plan.blocks_per_cu,
                 (long long)p->plan.workspace_bytes);
  }
  *plan_out = p;
  return RATTN_OK;
}

rattn_status rattn_plan_get_info(rattn_plan_t plan, rattn_plan_info* info) {
  if (plan == nullptr || info == nullptr) return RATTN_E_INVALID;
  fill_info(plan->prob, plan->plan, info);
  return RATTN_OK;
}

}  // extern "C"

namespace {

// One call's launches: the problem, its plan, the workspace that holds the split
// partials (plan.workspace_bytes bytes, the flag word in its last 256), and the flag
// word the kernels report bad device data in.
rattn_status decode_call(const rattn_problem& pr, const rattn::Plan& plan, void* workspace,
                         int32_t* flags, hipEvent_t* ev, const void* q, const void* k_cache,
                         const void* v_cache, const float* k_scale, const float* v_scale,
                         const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* cu_rows, int32_t row_cap, const float* bias, void* out,
                         float* lse, void* stream) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || page_table == nullptr ||
      seq_lens == nullptr || bias == nullptr || out == nullptr)
    return RATTN_E_INVALID;
  const bool fp8 = pr.kv_dtype == RATTN_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return RATTN_E_INVALID;

  rattn::KernelArgs a{};
  a.q = (const uint16_t*)q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.bias = bias;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.part_o = (float*)workspace;
  a.part_lse = a.part_o + plan.part_o_floats;
  a.unit_info = (int32_t*)(a.part_lse + plan.part_lse_floats);
  a.flags = flags;
  a.cu_rows = cu_rows;
  a.row_cap = row_cap;
  a.batch = pr.batch;
  a.n = pr.n_query_rows;
  a.num_q_heads = pr.num_q_heads;
  a.num_kv_heads = pr.num_kv_heads;
  a.group = pr.num_q_heads / pr.num_kv_heads;
  a.page_size = pr.page_size;
  a.page_shift = __builtin_ctz((unsigned)pr.page_size);
  a.num_pages = pr.num_pages;
  a.max_pages = pr.max_pages_per_seq;
  a.max_seq_len = pr.max_seq_len;
  a.window = pr.window;
  a.dmax = pr.dmax;
  a.softmax_scale = pr.softmax_scale;
  a.split_groups = plan.split_groups;
  a.splits_per_unit = plan.splits_per_unit;

  if (plan.prefill)
    return rattn::launch_prefill(a, plan.prefill_hw, a.group, fp8, stream, ev ? ev[0] : nullptr,
                                 ev ? ev[1] : nullptr) == 0
               ? RATTN_OK
               : RATTN_E_HIP;
  if (rattn::launch_split_kv(a, plan.waves, fp8, plan.ws, plan.rt, stream, ev ? ev[0] : nullptr,
                             ev ? ev[1] : nullptr) != 0)
    return RATTN_E_HIP;
  if (needs_combine(plan) &&
      rattn::launch_combine(a, stream, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr) != 0)
    return RATTN_E_HIP;
  return RATTN_OK;
}

rattn_status plan_call(rattn_plan_t plan, const void* q, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const int32_t* cu_rows, int32_t row_cap, const float* bias, void* out,
                       float* lse, void* stream) {
  if (plan == nullptr) return RATTN_E_INVALID;
  hipEvent_t* ev = nullptr;
  if (plan->prof_count < plan->prof_max && plan->prof_calls++ % plan->prof_stride == 0)
    ev = &plan->prof_events[4 * plan->prof_count++];
  return decode_call(plan->prob, plan->plan, plan->workspace, plan->flags, ev, q, k_cache,
                     v_cache, k_scale, v_scale, page_table, seq_lens, cu_rows, row_cap, bias,
                     out, lse, stream);
}

// Launch shape of the current device, for calls without a plan (rattn_decode_static):
// the CU count and, per split-kernel variant, the resident work-groups per CU, each
// queried once per device and kept.
struct DeviceShape {
  int cus = 0;
  int blocks_per_cu[64] = {};   // by variant: waves (1, 2, 4, 8) x format x partition
};
std::mutex g_shape_mutex;
DeviceShape g_shapes[64];

rattn_status device_shape(int dev, const rattn_problem& p, int32_t* cus, int32_t* bpc) {
  if (dev < 0 || dev >= 64) return RATTN_E_HIP;
  const int G = p.num_q_heads / p.num_kv_heads;
  const bool prefill = (int64_t)G * p.n_query_rows > rattn::kMaxRows;
  const rattn::SplitShape sh = prefill ? rattn::SplitShape{0, 1} : rattn::split_shape(p);
  const int waves = sh.waves, rt = sh.rt;
  const bool fp8 = p.kv_dtype == RATTN_KV_FP8_E4M3;
  const bool even = rattn::uses_even_shares(p);
  // layouts: one row tile in 1, 2, 4 or 8 waves (0-3); one wave of 2 or 3 row tiles
  // (4, 5); four waves of 2 (6)
  const int shape = rt > 1 ? (waves == 1 ? 2 + rt : 6)
                           : (waves == 8 ? 3 : waves == 4 ? 2 : waves == 2 ? 1 : 0);
  const int key = shape * 4 + (fp8 ? 2 : 0) + (even ? 1 : 0);
  std::lock_guard<std::mutex> lock(g_shape_mutex);
  DeviceShape& ds = g_shapes[dev];
  if (ds.cus == 0 &&
      hipDeviceGetAttribute(&ds.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    ds.cus = 0;
    return RATTN_E_HIP;
  }
  *cus = ds.cus;
  if (prefill) {
    *bpc = 1;
    return RATTN_OK;
  }
  if (ds.blocks_per_cu[key] == 0) {
    const int b = rattn::split_kv_blocks_per_cu(waves, fp8, even, rt);
    ds.blocks_per_cu[key] = b >= 1 ? b : rattn::kDefaultBlocksPerCU;
  }
  *bpc = ds.blocks_per_cu[key];
  return RATTN_OK;
}

}  // namespace

extern "C" {

rattn_status rattn_decode(rattn_plan_t plan, const void* q, const void* k_cache,
                          const void* v_cache, const float* k_scale, const float* v_scale,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const float* bias, void* out, float* lse, void* stream) {
  return plan_call(plan, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                   nullptr, 0, bias, out, lse, stream);
}

rattn_status rattn_decode_static(const rattn_problem* prob, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* page_table,
                                 const int32_t* seq_lens, const float* bias, void* out,
                                 float* lse, int32_t* flags, void* stream) {
  const rattn_status st = rattn::validate_problem(prob);
  if (st != RATTN_OK) return st;
  // pointer checks before any HIP call, as for rattn_decode
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || page_table == nullptr ||
      seq_lens == nullptr || bias == nullptr || out == nullptr)
    return RATTN_E_INVALID;
  const bool fp8 = prob->kv_dtype == RATTN_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return RATTN_E_INVALID;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RATTN_E_HIP;
  int32_t cus = 0, bpc = 0;
  if (device_shape(dev, *prob, &cus, &bpc) != RATTN_OK) return RATTN_E_HIP;
  const rattn::Plan plan = rattn::make_plan(*prob, cus, bpc);
  if (plan.workspace_bytes > rattn::kStaticScratchBytes) return RATTN_E_UNSUPPORTED;
  void* scratch = nullptr;    // this device's static array (resolved on its first call)
  if (rattn::static_scratch_ptr(dev, &scratch) != 0) return RATTN_E_HIP;
  // the flag word: the caller's, or the scratch's last 256 bytes (never read)
  int32_t* fl = flags != nullptr
                    ? flags
                    : (int32_t*)((char*)scratch + rattn::kStaticScratchBytes - 256);
  return decode_call(*prob, plan, scratch, fl, nullptr, q, k_cache, v_cache, k_scale, v_scale,
                     page_table, seq_lens, nullptr, 0, bias, out, lse, stream);
}

rattn_status rattn_decode_varlen(rattn_plan_t plan, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* page_table,
                                 const int32_t* seq_lens, const int32_t* cu_rows,
                                 int32_t num_rows, const float* bias, void* out, float* lse,
                                 void* stream) {
  if (plan == nullptr || cu_rows == nullptr || num_rows < 0) return RATTN_E_INVALID;
  if (plan->plan.prefill) return RATTN_E_UNSUPPORTED;   // rows per sequence: decode/verify
  return plan_call(plan, q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens,
                   cu_rows, num_rows, bias, out, lse, stream);
}

rattn_status rattn_append_kv(const rattn_problem* prob, const void* k_new, const void* v_new,
                             const int32_t* page_table, const int32_t* seq_lens, void* k_cache,
                             void* v_cache, float* k_scale, float* v_scale, int32_t* flags,
                             void* stream) {
  const rattn_status st = rattn::validate_problem(prob);
  if (st != RATTN_OK) return st;
  if (k_new == nullptr || v_new == nullptr || page_table == nullptr || seq_lens == nullptr ||
      k_cache == nullptr || v_cache == nullptr)
    return RATTN_E_INVALID;
  const bool fp8 = prob->kv_dtype == RATTN_KV_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return RATTN_E_INVALID;
  rattn::AppendArgs a{};
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.flags = flags;
  a.batch = prob->batch;
  a.n = prob->n_query_rows;
  a.num_kv_heads = prob->num_kv_heads;
  a.page_size = prob->page_size;
  a.page_shift = __builtin_ctz((unsigned)prob->page_size);
  a.num_pages = prob->num_pages;
  a.max_pages = prob->max_pages_per_seq;
  a.max_seq_len = prob->max_seq_len;
  a.fp8 = fp8 ? 1 : 0;
  return rattn::launch_append_kv(a, stream) == 0 ? RATTN_OK : RATTN_E_HIP;
}

rattn_status rattn_read_probe(const void* buf, int64_t nblocks, int32_t block_bytes,
                              const int32_t* order, int32_t waves, void* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || nblocks < 1 || block_bytes < 1024 ||
      block_bytes % 1024 != 0 || waves < 1 || waves > (1 << 20))
    return RATTN_E_INVALID;
  return rattn::launch_read_probe(buf, nblocks, block_bytes, order, waves, sink, stream) == 0
             ? RATTN_OK
             : RATTN_E_HIP;
}

rattn_status rattn_free(rattn_plan_t plan) {
  if (plan == nullptr) return RATTN_OK;
  destroy_events(plan);
  rattn_status st = RATTN_OK;
  if (plan->workspace != nullptr && hipFree(plan->workspace) != hipSuccess) st = RATTN_E_HIP;
  delete plan;
  return st;
}

rattn_status rattn_debug_flags(rattn_plan_t plan, int32_t* flags, void* stream) {
  if (plan == nullptr || flags == nullptr) return RATTN_E_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(flags, plan->flags, sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return RATTN_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return RATTN_E_HIP;
  if (hipMemsetAsync(plan->flags, 0, sizeof(int32_t), st) != hipSuccess) return RATTN_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return RATTN_E_HIP;
  return RATTN_OK;
}

rattn_status rattn_profile_begin(rattn_plan_t plan, int32_t max_calls, int32_t stride) {
  if (plan == nullptr || max_calls < 1 || max_calls > (1 << 20) || stride < 1)
    return RATTN_E_INVALID;
  destroy_events(plan);
  plan->prof_events.resize((size_t)4 * max_calls);
  for (size_t i = 0; i < plan->prof_events.size(); ++i) {
    // timing-only events, stamped by the kernel launches (no system-scope fence)
    if (hipEventCreateWithFlags(&plan->prof_events[i], hipEventDisableSystemFence) != hipSuccess) {
      plan->prof_events.resize(i);
      destroy_events(plan);
      return RATTN_E_HIP;
    }
  }
  plan->prof_max = max_calls;
  plan->prof_count = 0;
  plan->prof_stride = stride;
  plan->prof_calls = 0;
  return RATTN_OK;
}

rattn_status rattn_profile_end(rattn_plan_t plan, float* split_ms, float* combine_ms,
                               int32_t* ncalls) {
  if (plan == nullptr || split_ms == nullptr || combine_ms == nullptr || ncalls == nullptr)
    return RATTN_E_INVALID;
  const int32_t n = plan->prof_count;
  rattn_status st = RATTN_OK;
  for (int32_t i = 0; i < n && st == RATTN_OK; ++i) {
    hipEvent_t* ev = &plan->prof_events[4 * i];
    combine_ms[i] = 0.f;
    if (hipEventSynchronize(ev[1]) != hipSuccess ||
        hipEventElapsedTime(&split_ms[i], ev[0], ev[1]) != hipSuccess)
      st = RATTN_E_HIP;
    else if (needs_combine(plan->plan) &&
             (hipEventSynchronize(ev[3]) != hipSuccess ||
              hipEventElapsedTime(&combine_ms[i], ev[2], ev[3]) != hipSuccess))
      st = RATTN_E_HIP;
  }
  *ncalls = n;
  destroy_events(plan);
  return st;
}

}  // extern "C"
