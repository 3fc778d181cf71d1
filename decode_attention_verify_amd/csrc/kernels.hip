// HIP kernels for gfx950 (CDNA4): launchers and template instances.
//
//  * split_kv.h: split-KV relative-position GQA decode/verify attention over a piece of
//    each (sequence, KV head) unit's keys;
//  * combine.h: the log-sum-exp merge of the pieces of a unit that several work-groups
//    shared;
//  * append.h: the KV-cache write of each sequence's newest tokens, with E4M3
//    quantisation for an FP8 cache;
//  * prefill.h: the same attention for chunks of many query rows per sequence (chunked
//    prefill) over a bf16 cache, on the MFMA units; prefill_e4m3.h: over an E4M3 cache;
//  * probe.h: a streaming-read probe with the split kernel's load pattern (measurement);
//  * device_common.h: device helpers and the work partition.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "internal.h"
#include "append.h"
#include "combine.h"
#include "prefill.h"
#include "prefill_e4m3.h"
#include "probe.h"
#include "split_kv.h"

namespace rattn {

// ---------------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------------
// variant index: waves per piece (1, 2, 4, 8) of one row tile each, one wave of 2 or 3
// row tiles, or 4 waves of 2; KV format, partition; single-wave pieces also in merging
// groups of kMergeWaves
#define RATTN_VARIANTS(X)                                                               \
  X(1, false, false, 1) X(1, true, false, 1) X(2, false, false, 1) X(2, true, false, 1)  \
  X(4, false, false, 1) X(4, true, false, 1) X(8, false, false, 1) X(8, true, false, 1)  \
  X(1, false, true, 1) X(1, true, true, 1) X(2, false, true, 1) X(2, true, true, 1)      \
  X(4, false, true, 1) X(4, true, true, 1) X(8, false, true, 1) X(8, true, true, 1)      \
  X(1, false, false, 2) X(1, false, true, 2) X(1, false, false, 3) X(1, false, true, 3)      \
  X(4, false, false, 2) X(4, false, true, 2)

static int variant_key(int waves, bool fp8, bool even, int rt) {
  return (rt * 16 + waves) * 4 + (fp8 ? 2 : 0) + (even ? 1 : 0);
}

// A launch on `stream`; with events, through hipExtLaunchKernel, which stamps them with
// the kernel's own start and end (the timing of an instrumented call, without the
// stream gaps that events recorded around the launch would add).
template <typename Kernel, typename Args>
static int launch(Kernel kernel, dim3 grid, dim3 block, void* stream, const Args& a,
                  void* ev_start, void* ev_stop) {
  const hipStream_t st = (hipStream_t)stream;
  if (ev_start == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
    return (int)hipGetLastError();
  }
  Args copy = a;
  void* args[] = {&copy};
  return (int)hipExtLaunchKernel((const void*)kernel, grid, block, args, 0, st,
                                 (hipEvent_t)ev_start, (hipEvent_t)ev_stop, 0);
}

int launch_split_kv(const KernelArgs& a, int waves, bool fp8, int ws, int rt, void* stream,
                    void* ev_start, void* ev_stop) {
  const dim3 grid((unsigned)a.split_groups);
  if (ws > 1) {
    if (waves != 1 || fp8 || rt != 1 || a.splits_per_unit != ws) return (int)hipErrorInvalidValue;
    if (ws == 2)
      return launch(split_kv_kernel<1, false, false, 2, 1>, grid, dim3(128), stream, a, ev_start,
                    ev_stop);
    if (ws == 3)
      return launch(split_kv_kernel<1, false, false, 3, 1>, grid, dim3(192), stream, a, ev_start,
                    ev_stop);
    return (int)hipErrorInvalidValue;
  }
  if (ws != 1) return (int)hipErrorInvalidValue;
  const int key = variant_key(waves, fp8, a.splits_per_unit == 0, rt);
#define RATTN_LAUNCH(WRV, F8, EV, RTV)                                               \
  if (key == variant_key(WRV, F8, EV, RTV))                                          \
    return launch(split_kv_kernel<WRV, F8, EV, 1, RTV>, grid, dim3(64 * WRV), stream, a,  \
                  ev_start, ev_stop);
  RATTN_VARIANTS(RATTN_LAUNCH)
#undef RATTN_LAUNCH
  return (int)hipErrorInvalidValue;
}

int split_kv_blocks_per_cu(int waves, bool fp8, bool even, int rt) {
  const int key = variant_key(waves, fp8, even, rt);
  int nb = 0;
#define RATTN_OCC(WRV, F8, EV, RTV)                                                     \
  if (key == variant_key(WRV, F8, EV, RTV)) {                                           \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(                               \
               &nb, split_kv_kernel<WRV, F8, EV, 1, RTV>, 64 * WRV, 0) == hipSuccess     \
               ? nb                                                                     \
               : 0;                                                                     \
  }
  RATTN_VARIANTS(RATTN_OCC)
#undef RATTN_OCC
  return 0;
}

int launch_combine(const KernelArgs& a, void* stream, void* ev_start, void* ev_stop) {
  const int64_t rows = (int64_t)a.batch * a.n * a.num_q_heads;
  const dim3 grid((unsigned)combine_blocks(rows, a.splits_per_unit));
  switch (combine_shape(rows, a.splits_per_unit)) {
    case kCombineRows:
      return launch(combine_kernel<32, 2, 4, 8>, grid, dim3(256), stream, a, ev_start, ev_stop);
    case kCombineRows2:
      return launch(combine_kernel<32, 2, 4, 16>, grid, dim3(256), stream, a, ev_start, ev_stop);
    case kCombineWide:
      return launch(combine_kernel<8, 128, 1, 8>, grid, dim3(1024), stream, a, ev_start, ev_stop);
    case kCombineWide16:
      return launch(combine_kernel<4, 256, 1, 4>, grid, dim3(1024), stream, a, ev_start, ev_stop);
    default:
      return launch(combine_kernel<4, 16, 1, 8>, grid, dim3(64), stream, a, ev_start, ev_stop);
  }
}

int launch_prefill(const KernelArgs& a, int heads_per_wave, int group, bool fp8, void* stream,
                   void* ev_start, void* ev_stop) {
  const dim3 grid((unsigned)a.split_groups), block(64 * kPrefillWaves);
#define RATTN_PREFILL(HWV, HGV)                                                              \
  if (heads_per_wave == HWV && group == HWV * HGV)                                           \
    return fp8 ? launch(prefill_e4m3_kernel<HWV, HGV, kPrefillWaves>, grid, block, stream, a,  \
                        ev_start, ev_stop)                                                     \
               : launch(prefill_kernel<HWV, HGV, kPrefillWaves>, grid, block, stream, a,       \
                        ev_start, ev_stop);
  RATTN_PREFILL(3, 2) RATTN_PREFILL(2, 2) RATTN_PREFILL(2, 4)
#undef RATTN_PREFILL
  return (int)hipErrorInvalidValue;
}

int launch_read_probe(const void* buf, int64_t nblocks, int block_bytes, const int32_t* order,
                      int waves, void* sink, void* stream) {
  return launch(read_probe_kernel, dim3((unsigned)waves), dim3(64), stream,
                ProbeArgs{(const unsigned char*)buf, nblocks, block_bytes, order, (u32x4_t*)sink},
                nullptr, nullptr);
}

int launch_append_kv(const AppendArgs& a, void* stream) {
  const int64_t waves = (int64_t)2 * a.batch * a.n * a.num_kv_heads;
  return launch(append_kv_kernel, dim3((unsigned)waves), dim3(64), stream, a, nullptr, nullptr);
}

}  // namespace rattn
