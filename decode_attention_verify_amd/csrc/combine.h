// The log-sum-exp combine of the split kernel's partials.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"
#include "device_common.h"

namespace rattn {

// ---------------------------------------------------------------------------------
// Merge of the partials of a unit that several work-groups shared (page 2, FA4
// kernel: the KV range is split and merged): out = sum_s w_s O_s / sum_s w_s with
// w_s = exp(lse_s - max lse), and lse = max + ln sum w_s. Parts with lse = -inf (no
// visible key) are skipped.
//
// A thread (stripe, c4) of an output row merges pieces stripe, stripe + STRIPES, ...
// for dims 4 c4 .. 4 c4 + 3 of the row's slice with a running maximum, issuing the
// loads of UNROLL pieces at once (lse and O together), so that up to STRIPES * UNROLL
// pieces arrive in one memory round trip; the stripes are
// then merged by the same rule, with lane shuffles inside a wave and through LDS
// across the waves of a row. The shape follows the number of pieces:
//   * few pieces per unit: 64 lanes (2 stripes of 32) cover a whole row;
//   * tens of pieces: 16 stripes x 4 lanes per 16-dim slice of a row, one wave each;
//   * hundreds of pieces: 128 stripes x 8 lanes per 32-dim slice (or, for few rows,
//     256 x 4 per 16-dim slice), 16 waves (8 or 4 pieces in flight per thread, within
//     the 128 registers of a 1024-thread work-group).
// A unit held whole by one work-group was written by the split kernel and is left
// alone; a row that its sequence does not have is skipped.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void merge_part(float& m, float& l, f32x4_t& acc, float m2,
                                           float l2, f32x4_t acc2) {
  const float M = fmaxf(m, m2);
  const float w1 = m == kNegInf ? 0.f : __expf(m - M);
  const float w2 = m2 == kNegInf ? 0.f : __expf(m2 - M);
  l = l * w1 + l2 * w2;
  acc = acc * w1 + acc2 * w2;
  m = M;
}

template <int C4S, int STRIPES, int ROWS, int UNROLL>
__global__ __launch_bounds__(C4S * STRIPES * ROWS) void combine_kernel(KernelArgs a) {
  constexpr int SLICES = kHeadDim / (4 * C4S);           // work-group slices of a row
  constexpr int ROW_THREADS = C4S * STRIPES;
  constexpr int WAVES_PER_ROW = ROW_THREADS > 64 ? ROW_THREADS / 64 : 1;
  static_assert(ROWS == 1 || ROW_THREADS <= 64, "rows of a work-group stay within a wave");
  static_assert(ROW_THREADS % 64 == 0 || 64 % ROW_THREADS == 0, "rows tile the waves");
  __shared__ float red[WAVES_PER_ROW > 1 ? WAVES_PER_ROW * C4S * 6 : 1];

  const int t = threadIdx.x;
  const int c4 = t % C4S;
  const int stripe = (t / C4S) % STRIPES;
  const int64_t slot = (int64_t)blockIdx.x * ROWS + t / ROW_THREADS;
  const int64_t row = slot / SLICES;                     // slot (b * n + r) * Hq + h
  const int slice = (int)(slot - row * SLICES);
  const int Hq = a.num_q_heads;
  const int G = a.group;
  const int R = G * a.n;
  const int64_t rows = (int64_t)a.batch * a.n * Hq;
  const int64_t row_c = row < rows ? row : 0;            // a past-the-end slot reads row 0
  const int b = (int)(row_c / ((int64_t)a.n * Hq));
  const int rem = (int)(row_c - (int64_t)b * a.n * Hq);
  const int r = rem / Hq;
  const int h = rem - r * Hq;
  const int g = h / G;
  const int rho = r * G + (h - g * G);
  const SeqRows sr = seq_rows(a, b, false);
  const int64_t orow = (int64_t)(sr.base + r) * Hq + h;  // the row's place in out and lse

  const int64_t u = (int64_t)b * a.num_kv_heads + g;
  int64_t npieces, prow0;                                // piece k: row prow0 + k * R
  if (a.splits_per_unit > 0) {
    npieces = a.splits_per_unit;
    prow0 = u * npieces * R + rho;
  } else {
    npieces = a.unit_info[2 * u + 1];                    // recorded by the split kernel
    prow0 = (a.unit_info[2 * u] + u) * R + rho;
  }
  // nothing to merge: past the last row, a row the sequence does not have, or a unit
  // whose output its one work-group wrote (uniform over a row's threads)
  const bool live = row < rows && r < sr.n && npieces > 1;
  if (!live) npieces = 0;
  if (WAVES_PER_ROW == 1 && !live) return;               // no barrier in this shape

  float m = kNegInf, l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int dim0 = slice * 4 * C4S + 4 * c4;             // first dim of this thread
  for (int64_t k0 = stripe; k0 < npieces; k0 += STRIPES * UNROLL) {
    float ls[UNROLL];
    f32x4_t ov[UNROLL];
#pragma unroll
    for (int v = 0; v < UNROLL; ++v) {
      const int64_t k = k0 + STRIPES * v;
      ls[v] = k < npieces ? a.part_lse[prow0 + k * R] : kNegInf;
    }
    // the O loads do not wait for the lse loads: a piece past the last reads piece 0
    // again, and the O of an empty part (which its work-group never wrote) is dropped
    // after the load, so that both arrive in one memory round trip
#pragma unroll
    for (int v = 0; v < UNROLL; ++v) {
      const int64_t k = k0 + STRIPES * v;
      const int64_t kk = k < npieces ? k : 0;
      ov[v] = *reinterpret_cast<const f32x4_t*>(a.part_o + (prow0 + kk * R) * kHeadDim + dim0);
    }
#pragma unroll
    for (int v = 0; v < UNROLL; ++v) {
      if (ls[v] == kNegInf) continue;          // an empty part: its O is not used
      merge_part(m, l, acc, ls[v], 1.f, ov[v]);
    }
  }
  // the stripes of a wave
#pragma unroll
  for (int off = C4S; off < (ROW_THREADS < 64 ? ROW_THREADS : 64); off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    f32x4_t a2;
    a2[0] = __shfl_xor(acc[0], off);
    a2[1] = __shfl_xor(acc[1], off);
    a2[2] = __shfl_xor(acc[2], off);
    a2[3] = __shfl_xor(acc[3], off);
    merge_part(m, l, acc, m2, l2, a2);
  }
  bool writer = stripe == 0;
  if constexpr (WAVES_PER_ROW > 1) {
    // the waves of a row: lanes 0 .. C4S-1 of each wave hold its result; wave 0 merges
    // them, lane (j, c4) taking waves j, j + 64 / C4S, ... before a last shuffle merge
    constexpr int J = 64 / C4S;
    const int wave = t >> 6, lane = t & 63;
    if (lane < C4S) {
      float* e = red + (wave * C4S + lane) * 6;
      e[0] = m; e[1] = l; e[2] = acc[0]; e[3] = acc[1]; e[4] = acc[2]; e[5] = acc[3];
    }
    __syncthreads();
    writer = false;
    if (wave == 0) {
      m = kNegInf; l = 0.f; acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int w = lane / C4S; w < WAVES_PER_ROW; w += J) {
        const float* e = red + (w * C4S + c4) * 6;
        merge_part(m, l, acc, e[0], e[1], f32x4_t{e[2], e[3], e[4], e[5]});
      }
#pragma unroll
      for (int off = C4S; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off);
        const float l2 = __shfl_xor(l, off);
        f32x4_t a2;
        a2[0] = __shfl_xor(acc[0], off);
        a2[1] = __shfl_xor(acc[1], off);
        a2[2] = __shfl_xor(acc[2], off);
        a2[3] = __shfl_xor(acc[3], off);
        merge_part(m, l, acc, m2, l2, a2);
      }
      writer = lane < C4S;
    }
    if (!live) return;
  }
  if (writer) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const f32x4_t v = acc * inv;
    const u32x2_t wv = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2_t*>(a.out + orow * kHeadDim + dim0) = wv;
    if (dim0 == 0 && a.lse != nullptr) a.lse[orow] = l > 0.f ? m + __logf(l) : kNegInf;
  }
}

}  // namespace rattn
