// Device helpers shared by the kernels: vector types, streaming loads, bf16 packing, the
// exact E4M3 decode, row reductions, LDS swizzles, and the work partition of the split
// kernel (which the combine reads back).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace rattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 5.545177444479562f;   // 8 ln 2: p = exp(s - m) <= 256
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Streaming loads for data that one call reads exactly once (K/V pages, their scales,
// bias entries): the non-temporal hint keeps them from displacing reusable lines and,
// measured on MI355X over permuted 4 KiB pages, raises the sustained read rate from
// about 5.7 to 6.4 TB/s.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ f32x4_t ldf4_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}

__device__ __forceinline__ float ldf_stream(const float* p) {
  return __builtin_nontemporal_load(p);
}

// Four adjacent floats at any 4-byte aligned address. The type's 4-byte alignment keeps
// the access defined: the compiler emits one 16-byte load where the target allows
// unaligned dword-multiple accesses, else four 4-byte loads.
typedef float f32x4u_t __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ f32x4_t ldf4u_stream(const float* p) {
  const f32x4u_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4u_t*>(p));
  return f32x4_t{v[0], v[1], v[2], v[3]};
}

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// What pack_bf16x2(lo, hi) = `packed` left out, rounded to bf16 in turn: the pair
// `packed` + this remainder carries lo and hi to about 2^-17 of their size (a P scaled
// by an E4M3 value scale goes to the matrix units as these two bf16 parts).
__device__ __forceinline__ unsigned int pack_bf16x2_rem(float lo, float hi, unsigned int packed) {
  return pack_bf16x2(lo - __uint_as_float(packed << 16), hi - __uint_as_float(packed & 0xffff0000u));
}

// Four E4M3 codes (one dword) -> four bf16 values (two dwords), in code order. Exact:
// every E4M3 value, subnormals included, is a bf16 value. v_cvt_scalef32_pk_bf16_fp8
// (gfx950) converts two codes per instruction (scale 1); checked on MI355X against the
// format's definition for all 256 codes, NaN codes included.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(unsigned int w) {
  u32x2_t r;
  r.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// The 4 lanes lr, lr+16, lr+32, lr+48 hold the same query row. The gfx950 permlane
// swaps exchange their values inside the VALU, without an LDS round trip: a 16-lane
// swap of a value with itself leaves lane l holding its own value and that of lane
// l ^ 16 (one in each result, in an order that depends on l), a 32-lane swap that of
// lane l ^ 32.
template <int SPAN>
__device__ __forceinline__ void lane_pair(float x, float& p, float& q) {
  const unsigned u = __float_as_uint(x);
  const auto r = SPAN == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                            : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  p = __uint_as_float(r[0]);
  q = __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_rows(float x) {
  float p, q;
  lane_pair<16>(x, p, q);
  x = fmaxf(p, q);
  lane_pair<32>(x, p, q);
  return fmaxf(p, q);
}

__device__ __forceinline__ float wave_sum_rows(float x) {
  float p, q;
  lane_pair<16>(x, p, q);
  x = p + q;
  lane_pair<32>(x, p, q);
  return p + q;
}

// Byte offset in the LDS V tile of 16-byte chunk `cc` (0..15) of key row `k` (0..31).
// Rows are 256 bytes; the chunk index is XOR-swizzled by the row so that the 16 rows
// one transpose read touches fall into distinct banks.
// Byte offset in the LDS K tile of 16-byte chunk `c` (0..15) of key row `k` (0..31):
// the chunk is XOR-swizzled by the row's low 4 bits, so the 16 lanes of one pass of a
// 16-byte LDS access (one row written, or 16 rows read at one chunk) hit distinct banks.
__device__ __forceinline__ int klds_off(int k, int c) {
  return k * 256 + ((c ^ (k & 15)) << 4);
}

__device__ __forceinline__ int vlds_off(int k, int cc) {
  return k * 256 + ((cc ^ ((k & 7) << 1)) << 4);
}

// ---------------------------------------------------------------------------------
// Work partition. Sequence b contributes, for each of its KV heads, the 32-key tiles
// of its visible range [base_b, L_b); a (sequence, KV head) pair is a unit. Two ways of
// sharing the units among the split work-groups:
//  * per unit (splits_per_unit = k > 0): work-group w takes the s-th of k near-equal
//    tile ranges of unit u = w / k (s = w % k); its partials live under piece id w.
//    Suits units of equal length (batch-1 decode, sliding-window layers).
//  * evenly (k = 0): the (sequence, KV head, tile) space, sequences outermost, is cut
//    into P equal contiguous shares. A share may cover the end of one unit and the
//    start of the next: each such piece is attended separately and its partial lives
//    under the piece id w + u, which is unique because walking the tile axis advances
//    w, u or both at every piece boundary. Suits batches of very different lengths.
// A work-group whose piece is a whole unit writes the final output itself.
// ---------------------------------------------------------------------------------
// The query rows of sequence b: n each at rows b*n .., or the packed range that
// cu_rows gives (at most n rows, within the row buffers; else none, flagged).
struct SeqRows {
  int base;    // row index of the sequence's first query row in q, out and lse
  int n;       // its rows, the last n positions of the sequence
};

__device__ __forceinline__ SeqRows seq_rows(const KernelArgs& a, int b, bool flag_bad) {
  if (a.cu_rows == nullptr) return SeqRows{b * a.n, a.n};
  const int lo = a.cu_rows[b], hi = a.cu_rows[b + 1];
  if (lo < 0 || hi < lo || hi - lo > a.n || hi > a.row_cap) {
    if (flag_bad) atomicOr(a.flags, RATTN_FLAG_ROWS_INVALID);
    return SeqRows{0, 0};
  }
  return SeqRows{lo, hi - lo};
}

struct SeqGeom {
  int nb;      // query rows of the sequence
  int L;       // length (clamped into [nb, max_seq_len])
  int k_lo;    // first key visible to the earliest query row
  int base;    // k_lo rounded down to a tile boundary
  int tiles;   // tiles of [base, L); none for a sequence without rows
};

__device__ __forceinline__ SeqGeom seq_geom(const KernelArgs& a, int b, int nb, bool flag_bad) {
  int L = a.seq_lens[b];
  if (L < nb || L > a.max_seq_len) {
    if (flag_bad) atomicOr(a.flags, RATTN_FLAG_SEQ_LEN_CLAMPED);
    L = min(max(L, nb), a.max_seq_len);
  }
  SeqGeom g;
  g.nb = nb;
  g.L = L;
  g.k_lo = a.window > 0 ? max(0, L - nb + 1 - a.window) : 0;
  g.base = g.k_lo & ~(kTileKeys - 1);
  g.tiles = nb > 0 ? (L - g.base + kTileKeys - 1) / kTileKeys : 0;
  return g;
}

__device__ __forceinline__ SeqGeom seq_geom(const KernelArgs& a, int b, bool flag_bad) {
  return seq_geom(a, b, seq_rows(a, b, flag_bad).n, flag_bad);
}

// Tiles of all units (every lane returns the total; below 2^31 by validation).
__device__ int total_tiles(const KernelArgs& a, int lane) {
  int sum = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int b = b0 + lane;
    int v = b < a.batch ? seq_geom(a, b, true).tiles * a.num_kv_heads : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    sum += v;
  }
  return sum;
}

// The sequence whose units hold tile t (t < total), and the tiles before it.
__device__ void locate_tile(const KernelArgs& a, int lane, int t, int& b_out, int& before_out) {
  int carry = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int b = b0 + lane;
    const int v = b < a.batch ? seq_geom(a, b, false).tiles * a.num_kv_heads : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int chunk = __shfl(incl, 63);
    if (t < carry + chunk) {                                 // uniform
      const unsigned long long hit = __ballot(carry + incl > t);
      const int idx = __ffsll(hit) - 1;
      b_out = b0 + idx;
      before_out = carry + __shfl(incl - v, idx);
      return;
    }
    carry += chunk;
  }
  b_out = a.batch - 1;                                       // not reached for t < total
  before_out = carry;
}

}  // namespace rattn
