// The KV-cache append with E4M3 quantisation.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"
#include "device_common.h"

namespace rattn {

// ---------------------------------------------------------------------------------
// KV-cache append (the step just before the attention; page 3, section on speeding up
// the implementation: a fused KV-cache update; page 2's roadmap and page 3's support
// section: an FP8 KV cache). One wave per (K or V, sequence, new token, KV head): token
// r of sequence b sits at position t = L_b - n + r, slot t mod S of page
// page_table[b][t div S]. A bf16 cache gets the row as given. An E4M3 cache gets the
// codes of clamp(x / s, +-448) with s = max|x| / 448 (1 for an all-zero row), both
// quotients correctly rounded in fp32, rounded to the nearest code (ties to even) by
// v_cvt_pk_fp8_f32, and the scale s.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_kv_kernel(AppendArgs a) {
  const int lane = threadIdx.x;
  int64_t id = blockIdx.x;
  const int g = (int)(id % a.num_kv_heads);
  id /= a.num_kv_heads;
  const int r = (int)(id % a.n);
  id /= a.n;
  const int b = (int)(id % a.batch);
  const int kv = (int)(id / a.batch);            // 0: K, 1: V

  const int L = a.seq_lens[b];
  if (L < a.n || L > a.max_seq_len) {            // nothing is written for a bad length
    if (lane == 0 && a.flags != nullptr) atomicOr(a.flags, RATTN_FLAG_SEQ_LEN_CLAMPED);
    return;
  }
  const int t = L - a.n + r;
  const int ph = a.page_table[(int64_t)b * a.max_pages + (t >> a.page_shift)];
  if (ph < 0 || ph >= a.num_pages) {             // nor for a page id outside the cache
    if (lane == 0 && a.flags != nullptr) atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
    return;
  }
  const int64_t row = ((int64_t)ph * a.num_kv_heads + g) * a.page_size + (t & (a.page_size - 1));
  const uint16_t* src = (kv ? a.v_new : a.k_new) +
                        (((int64_t)b * a.n + r) * a.num_kv_heads + g) * kHeadDim;
  const unsigned pair = *reinterpret_cast<const unsigned*>(src + 2 * lane);   // dims 2l, 2l+1
  if (!a.fp8) {
    uint16_t* dst = (uint16_t*)(kv ? a.v_cache : a.k_cache) + row * kHeadDim;
    *reinterpret_cast<unsigned*>(dst + 2 * lane) = pair;
    return;
  }
  const float x0 = __builtin_bit_cast(float, pair << 16);
  const float x1 = __builtin_bit_cast(float, pair & 0xffff0000u);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
  const float y0 = fminf(fmaxf(x0 / s, -kE4M3Max), kE4M3Max);
  const float y1 = fminf(fmaxf(x1 / s, -kE4M3Max), kE4M3Max);
  const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);   // bytes 0, 1
  unsigned char* dst = (unsigned char*)(kv ? a.v_cache : a.k_cache) + row * kHeadDim;
  *reinterpret_cast<uint16_t*>(dst + 2 * lane) = (uint16_t)(codes & 0xffff);
  if (lane == 0) (kv ? a.v_scale : a.k_scale)[row] = s;
}

}  // namespace rattn
