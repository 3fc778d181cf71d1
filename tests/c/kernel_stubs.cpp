// Stand-ins for the device-side launchers (kernels.hip, scratch.hip), so that the host
// library (api.cpp, planner.cpp) can be built with the host compiler alone and run
// under the address and undefined-behaviour sanitizers on a machine without a GPU.
// Every launch reports failure; the occupancy query reports the gfx950 default.
#include "../../decode_attention_verify_amd/csrc/internal.h"

namespace rattn {

int launch_split_kv(const KernelArgs&, int, bool, int, int, void*, void*, void*) { return 1; }
int launch_combine(const KernelArgs&, void*, void*, void*) { return 1; }
int launch_append_kv(const AppendArgs&, void*) { return 1; }
int launch_prefill(const KernelArgs&, int, int, bool, void*, void*, void*) { return 1; }
int launch_read_probe(const void*, int64_t, int, const int32_t*, int, void*, void*) { return 1; }
int split_kv_blocks_per_cu(int, bool, bool, int) { return kDefaultBlocksPerCU; }
int static_scratch_ptr(int, void** ptr) {
  *ptr = nullptr;
  return 1;
}

}  // namespace rattn
