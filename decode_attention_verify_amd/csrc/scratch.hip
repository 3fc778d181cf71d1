// Device memory for calls that must not allocate (rattn_decode_static): one static
// array, which the code object gives every GPU the library runs on, holding the split
// partials, the unit records and the flag word of such a call.
//
// Host code never names the array itself except to resolve its address: in host code
// `scratch` is a stand-in, not a device address. Each device's address is resolved once,
// with that device current, by hipGetSymbolAddress, and kept; kernels receive that
// address through their arguments.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace rattn {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];     // per device; null until resolved

}  // namespace

int static_scratch_ptr(int device, void** ptr) {
  if (ptr == nullptr) return (int)hipErrorInvalidValue;
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    int current = -1;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return (int)e;
    if (current != device) return (int)hipErrorInvalidDevice;   // resolve on `device` only
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return 0;
}

}  // namespace rattn
