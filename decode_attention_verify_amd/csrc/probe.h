// A measurement aid, not part of the attention: streams the blocks of a buffer in a
// given order with the split kernel's load pattern (non-temporal 16-byte loads, each
// 64-lane pass reading 1 KiB of contiguous bytes, two blocks in flight per wave), so
// that a benchmark can report the read rate this access pattern reaches on the device
// beside the nominal HBM peak.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"
#include "device_common.h"

namespace rattn {

struct ProbeArgs {
  const unsigned char* buf;    // nblocks blocks of block_bytes (a multiple of 1 KiB)
  int64_t nblocks;
  int block_bytes;
  const int32_t* order;        // the order to read the blocks in (null: in place order)
  u32x4_t* sink;               // 64 x 16 bytes
};

__global__ __launch_bounds__(64) void read_probe_kernel(ProbeArgs a) {
  const unsigned char* buf = a.buf;
  const int64_t nblocks = a.nblocks;
  const int block_bytes = a.block_bytes;
  const int32_t* order = a.order;
  const int lane = threadIdx.x;
  const int64_t per = (nblocks + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = min(b0 + per, nblocks);
  const int passes = block_bytes >> 10;                  // 1 KiB per 64-lane pass
  u32x4_t acc = {0, 0, 0, 0};
  auto block_at = [&](int64_t b) -> const unsigned char* {
    int64_t k = order != nullptr ? (int64_t)order[b] : b;
    k = k < 0 ? 0 : (k >= nblocks ? nblocks - 1 : k);      // a bad entry reads a valid block
    return buf + k * block_bytes + 16 * lane;
  };
  for (int64_t b = b0; b < b1; b += 2) {
    const unsigned char* p = block_at(b);
    const unsigned char* q = block_at(min(b + 1, b1 - 1));
    for (int s = 0; s < passes; s += 4) {
      u32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ss = min(s + u, passes - 1);
        v[u] = ld16_stream(p + 1024 * ss);
        v[4 + u] = ld16_stream(q + 1024 * ss);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
  }
  // a write the compiler cannot rule out keeps the loads; it practically never happens
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) a.sink[lane] = acc;
}

}  // namespace rattn
