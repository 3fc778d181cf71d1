// HIP kernels for gfx950 (CDNA4): split-KV relative-position GQA decode/verify
// attention and the log-sum-exp combine of its partials.
//
// Method (page 2 "vLLM TML Inkling support", model architecture section): logits
// s_j = scale * q.k_j + B[h][min(p - j, Dmax)], softmax over the visible keys. Page 1
// ("vLLM supports Inkling 2 Small", section on vLLM's optimisations) packs the 6 query
// heads of a GQA group into one tile so that each K/V page is read once per group;
// page 2 (technical optimisations, FA4 kernel) splits the KV range, with a "sheared"
// bias access, and merges the splits.
//
// Design on gfx950:
//  * one wave64 work-group per (split, KV head, sequence);
//  * the G*n query rows of the group (G = Hq/Hkv) are packed into 16-row MFMA tiles
//    (6 rows pad to 16 here, not to 64 as in the pages' Blackwell tile);
//  * S^T = K * Q^T on v_mfma_f32_16x16x32_bf16 with K as the A operand, loaded straight
//    from HBM into registers in the MFMA operand layout (each lane reads 16 contiguous
//    bytes of one key row; no LDS round trip for K);
//  * the S^T accumulator layout (lane = query row, 4 keys per lane) is exactly the B
//    operand layout that O^T = V^T * P^T needs, so P never moves between lanes;
//  * V is staged through LDS (XOR-swizzled 16-byte chunks) and read back transposed
//    with ds_read_b64_tr_b16, the gfx950 LDS transpose read;
//  * the bias is read per lane as 4 consecutive distances, shifted by one per verify
//    row (the sheared access): each row of a head reads the same slice one float over;
//  * online softmax in fp32, one row per lane, row max across the 4 lanes of a row;
//  * FP8 (OCP E4M3) K/V are decoded exactly to bf16 with v_cvt_pk_f32_fp8; the K scale
//    multiplies the logit column, the V scale multiplies P before its bf16 rounding.
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

__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (unsigned int)__builtin_bit_cast(unsigned short, a) |
         ((unsigned int)__builtin_bit_cast(unsigned short, b) << 16);
}

// Four E4M3 codes (one dword) -> four bf16 values (two dwords). Exact: every E4M3
// value, subnormals included, is a bf16 value, so the bf16 word is the upper half of
// the fp32 word that v_cvt_pk_f32_fp8 produces.
// The packed result is bit-cast to two dwords as a whole before its halves are used:
// this compiler folds a float element extracted from that builtin's float2 result into
// the other element (element y read as x), which the whole-vector bit cast avoids.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(unsigned int w) {
  const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false));
  const u32x2_t hi = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true));
  u32x2_t r;
  r.x = __builtin_amdgcn_perm(lo.y, lo.x, 0x07060302u);   // {bf16(b0), bf16(b1)}
  r.y = __builtin_amdgcn_perm(hi.y, hi.x, 0x07060302u);   // {bf16(b2), bf16(b3)}
  return r;
}

// The 4 lanes lr, lr+16, lr+32, lr+48 hold the same query row. (The gfx950 permlane
// swaps would keep this in the VALU, but this compiler folds the two results of a swap
// whose operands are the same value into one, so the reductions use lane shuffles.)
__device__ __forceinline__ float wave_max_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
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

template <int NRT, bool FP8>
__global__ __launch_bounds__(64) void split_kv_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char klds[kTileKeys * 256];
  __shared__ __attribute__((aligned(16))) unsigned char vlds[kTileKeys * 256];
  __shared__ int pages_lds[kChunkPages + 1];

  const int lane = threadIdx.x;
  const int lr = lane & 15;        // key (A operand) / query row (B operand) within a tile
  const int lq = lane >> 4;        // k-group of the MFMA operands
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int n = a.n;
  const int G = a.group;
  const int R = G * n;
  const int S = a.page_size;

  int L = a.seq_lens[b];
  if (L < n || L > a.max_seq_len) {
    if (lane == 0) atomicOr(a.flags, RATTN_FLAG_SEQ_LEN_CLAMPED);
    L = min(max(L, n), a.max_seq_len);
  }
  const int W = a.window;
  const int k_lo = W > 0 ? max(0, L - n + 1 - W) : 0;
  const int base = k_lo & ~(kTileKeys - 1);
  const int j_begin = base + split * a.keys_per_split;
  if (j_begin >= L) {
    // an empty split (a short sequence in a batch planned for longer ones) marks its
    // rows with lse = -inf, which the combine skips
    if (a.num_splits > 1) {
      for (int rho = lane; rho < R; rho += 64) {
        const int r = rho / G;
        const int64_t row = (int64_t)(b * n + r) * a.num_q_heads + g * G + (rho - r * G);
        a.part_lse[row * a.num_splits + split] = kNegInf;
      }
    }
    return;
  }
  const int j_end = min(j_begin + a.keys_per_split, L);
  // tiles at or after `fast_lo` and before `fast_hi` need no mask: every key is
  // visible to every row at a distance in [0, W-1]
  const int fast_lo = W > 0 ? max(0, L - W) : 0;
  const int fast_hi = L - n - (kTileKeys - 1);   // j0 <= fast_hi
  // tiles with bias_lo <= j0 <= fast_hi see only distances in [0, Dmax]: their bias
  // entries are addressed without clamping
  const int bias_lo = L - 1 - a.dmax;

  // ---- the packed query rows of this lane (row rho = 16 t + lr) ----
  int row_h[NRT], row_p[NRT];
  bool row_ok[NRT];
  bf16x8_t qreg[NRT][4];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const int rho = 16 * t + lr;
    row_ok[t] = rho < R;
    const int r = row_ok[t] ? rho / G : 0;
    const int hl = row_ok[t] ? rho - r * G : 0;
    row_h[t] = g * G + hl;
    row_p[t] = L - n + r;
    const uint16_t* qrow = a.q + ((int64_t)(b * n + r) * a.num_q_heads + row_h[t]) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // the K operand of MFMA s gives lane (lr, lq) the dims 32 s + 8 lq .. + 7
      const int d0 = 32 * s + 8 * lq;
      u32x4_t v = row_ok[t] ? ld16(qrow + d0) : u32x4_t{0, 0, 0, 0};
      qreg[t][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // bias entry of this lane's row at distance row_p - 4 lq - j, as an element offset
  // from the table start once j is subtracted (the table has fewer than 2^31 entries)
  int bias_row[NRT], bias_off[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    bias_row[t] = row_h[t] * (a.dmax + 1);
    bias_off[t] = bias_row[t] + row_p[t] - 4 * lq;
  }

  // ---- page ids ----
  // The ids of the pages a chunk of the split touches are staged in LDS before its tile
  // loop, so that the loop looks them up with an LDS read: a page-table load inside the
  // loop would make every tile wait for all of its predecessors' K/V loads.
  const int32_t* pt_row = a.page_table + (int64_t)b * a.max_pages;
  int chunk_p0 = 0;
  auto stage_pages = [&](int c0, int c1) {
    chunk_p0 = c0 >> a.page_shift;
    const int np = ((c1 - 1) >> a.page_shift) - chunk_p0 + 1;   // <= kChunkPages + 1
    for (int i = lane; i < np; i += 64) {
      int ph = pt_row[chunk_p0 + i];
      if (ph < 0 || ph >= a.num_pages) {
        atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
        ph = min(max(ph, 0), a.num_pages - 1);
      }
      pages_lds[i] = ph;
    }
  };
  auto phys_at = [&](int jt) -> int {      // physical page of key jt of the current chunk
    const int idx = min(max((jt >> a.page_shift) - chunk_p0, 0), kChunkPages);
    return __builtin_amdgcn_readfirstlane(pages_lds[idx]);
  };

  // ---- per-tile registers ----
  constexpr int KV_REGS = FP8 ? 2 : 4;   // 16-byte loads per lane per subtile (K)
  constexpr int V_LOADS = FP8 ? 4 : 8;   // 16-byte loads per lane per tile (V)
  struct Tile {
    u32x4_t k[2][KV_REGS];
    u32x4_t v[V_LOADS];
    f32x4_t ks[2], vs[2];
    float bias[NRT][2][4];
  };

  const int64_t Hkv = a.num_kv_heads;
  const int sub_lo = k_lo & ~15;         // first 16-key subtile holding a visible key
  const int sub_hi = (L - 1) & ~15;      // last subtile holding a key of the sequence
  // Every load of a tile is issued unconditionally, so that the compiler can count the
  // loads in flight and wait for exactly one tile at a time. A subtile with no key in
  // [k_lo, L) (at the two ends of the visible range) reads the nearest subtile that has
  // one instead; the masks of process_tile discard its keys.
  // 32-bit lane offsets from a page's (uniform) base address, so that the loads take
  // the scalar-base + vector-offset form and need no per-tile address arithmetic
  constexpr int ROW_BYTES = FP8 ? kHeadDim : 2 * kHeadDim;
  const unsigned kv_off = FP8 ? (lane >> 3) * 128 + 16 * (lane & 7) : lq * 256 + 16 * lr;
  const unsigned sc_off = 16 * lq;
  const unsigned char* kc = (const unsigned char*)a.k_cache;
  const unsigned char* vc = (const unsigned char*)a.v_cache;
  auto load_tile = [&](Tile& T, int j0) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int jt = j0 + 16 * kt;
      const int js = min(max(jt, sub_lo), sub_hi);
      const int ph = phys_at(js);
      const int64_t tok0 = ((int64_t)ph * Hkv + g) * S + (js & (S - 1));
      const unsigned char* kb = kc + tok0 * ROW_BYTES;
      const unsigned char* vb = vc + tok0 * ROW_BYTES;
      // K and V alike: each 16-lane pass of a load reads 256 contiguous bytes (one bf16
      // row, two E4M3 rows); a pass spread over 16 rows caps the read rate near 5.2 TB/s
      if (!FP8) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {    // keys 4u + lq of this subtile, chunk lr
          T.k[kt][u] = ld16_stream(kb + kv_off + 1024 * u);
          T.v[4 * kt + u] = ld16_stream(vb + kv_off + 1024 * u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {    // keys 8u + lane/8 of this subtile, chunk lane%8
          T.k[kt][u] = ld16_stream(kb + kv_off + 1024 * u);
          T.v[2 * kt + u] = ld16_stream(vb + kv_off + 1024 * u);
        }
        const unsigned char* ksb = (const unsigned char*)(a.k_scale + tok0);
        const unsigned char* vsb = (const unsigned char*)(a.v_scale + tok0);
        T.ks[kt] = __builtin_nontemporal_load((const f32x4_t*)(ksb + sc_off));
        T.vs[kt] = __builtin_nontemporal_load((const f32x4_t*)(vsb + sc_off));
      }
    }
    // bias: row r of head h reads B[h][p_r - j] for its 4 keys; rows of one head read
    // the same slice shifted by their offset r (the sheared access)
    if (j0 >= bias_lo && j0 <= fast_hi) {       // uniform: no clamping needed
      const unsigned char* bb = (const unsigned char*)a.bias;
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
        const unsigned o = (unsigned)(bias_off[t] - j0) * 4u;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            T.bias[t][kt][i] = __builtin_nontemporal_load(
                (const float*)(bb + o - 4 * (16 * kt + i)));
      }
    } else {                                    // distances clamped to [0, Dmax]
#pragma unroll
      for (int t = 0; t < NRT; ++t)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int dist = row_p[t] - (j0 + 16 * kt + 4 * lq + i);
            dist = min(max(dist, 0), a.dmax);
            T.bias[t][kt][i] = ldf_stream(a.bias + (unsigned)(bias_row[t] + dist));
          }
    }
  };

  // ---- running state ----
  f32x4_t o[NRT][8];
  float m_run[NRT], l_run[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    m_run[t] = kNegInf;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4_t{0, 0, 0, 0};
  }

  auto process_tile = [&](const Tile& T, int j0) {
    const bool fast = (j0 >= fast_lo) && (j0 <= fast_hi);   // uniform

    // V -> LDS (bf16, swizzled); keys outside [k_lo, L) become zero so that P = 0
    // times a stale or NaN value cannot reach the accumulator
    if (!FP8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = 4 * u + lq;
        const int j = j0 + kk;
        u32x4_t v = T.v[u];
        if (!fast && (j < k_lo || j >= L)) v = u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t*>(vlds + vlds_off(kk, lr)) = v;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = 8 * u + (lane >> 3);
        const int j = j0 + kk;
        const int c8 = lane & 7;
        u32x4_t raw = T.v[u];
        if (!fast && (j < k_lo || j >= L)) raw = u32x4_t{0, 0, 0, 0};
        u32x2_t a0 = e4m3x4_to_bf16x4(raw.x), a1 = e4m3x4_to_bf16x4(raw.y);
        u32x2_t a2 = e4m3x4_to_bf16x4(raw.z), a3 = e4m3x4_to_bf16x4(raw.w);
        *reinterpret_cast<u32x4_t*>(vlds + vlds_off(kk, 2 * c8)) =
            u32x4_t{a0.x, a0.y, a1.x, a1.y};
        *reinterpret_cast<u32x4_t*>(vlds + vlds_off(kk, 2 * c8 + 1)) =
            u32x4_t{a2.x, a2.y, a3.x, a3.y};
      }
    }

    // K -> LDS as bf16 (swizzled), then the MFMA A operands: lane (lr, lq) of MFMA s
    // reads key 16 kt + lr, dims 32 s + 8 lq .. + 7
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (!FP8) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          *reinterpret_cast<u32x4_t*>(klds + klds_off(16 * kt + 4 * u + lq, lr)) = T.k[kt][u];
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kk = 16 * kt + 8 * u + (lane >> 3);
          const int c8 = lane & 7;
          const u32x4_t raw = T.k[kt][u];
          u32x2_t c0 = e4m3x4_to_bf16x4(raw.x), c1 = e4m3x4_to_bf16x4(raw.y);
          u32x2_t c2 = e4m3x4_to_bf16x4(raw.z), c3 = e4m3x4_to_bf16x4(raw.w);
          *reinterpret_cast<u32x4_t*>(klds + klds_off(kk, 2 * c8)) = u32x4_t{c0.x, c0.y, c1.x, c1.y};
          *reinterpret_cast<u32x4_t*>(klds + klds_off(kk, 2 * c8 + 1)) =
              u32x4_t{c2.x, c2.y, c3.x, c3.y};
        }
      }
    }
    // S^T = K Q^T : lane holds row lr (+16 t), keys 4 lq + i of each 16-key subtile
    bf16x8_t kop[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kop[kt][s] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(klds + klds_off(16 * kt + lr, 4 * s + lq)));
    f32x4_t sacc[NRT][2];
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt][s], qreg[t][s], acc, 0, 0, 0);
        sacc[t][kt] = acc;
      }
    }

    // logits, mask, online softmax; P packed as the B operand of O^T += V^T P^T
    bf16x8_t pop[NRT];
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      float sv[2][4];
      float mt = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float scl = FP8 ? a.softmax_scale * T.ks[kt][i] : a.softmax_scale;
          float s = __builtin_fmaf(sacc[t][kt][i], scl, T.bias[t][kt][i]);
          if (!fast) {
            const int dist = row_p[t] - (j0 + 16 * kt + 4 * lq + i);
            const bool vis = row_ok[t] && dist >= 0 && (W == 0 || dist < W);
            s = vis ? s : kNegInf;
          }
          sv[kt][i] = s;
          mt = fmaxf(mt, s);
        }
      }
      mt = wave_max_rows(mt);
      // The reference point m of a row moves only when the tile's maximum exceeds it by
      // more than kRescaleSlack, so that the accumulators are rescaled on few tiles;
      // p = exp(s - m) then stays below exp(kRescaleSlack). O and l share m, so the
      // quotient O / l and lse = m + ln l are unchanged by the choice of m.
      const bool grow = mt > m_run[t] + kRescaleSlack;    // false while mt = -inf
      if (__ballot(grow) != 0) {                          // wave-uniform
        const float m_new = grow ? mt : m_run[t];
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run[t] - m_new) * kLog2e) : 1.f;
        l_run[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
        m_run[t] = m_new;
      }
      const float m_use = m_run[t] == kNegInf ? 0.f : m_run[t];
      const float mb = -m_use * kLog2e;
      float psum = 0.f;
      float pv[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kt][i], kLog2e, mb));
          psum += p;
          pv[kt][i] = FP8 ? (p > 0.f ? p * T.vs[kt][i] : 0.f) : p;
        }
      }
      l_run[t] += psum;
      u32x4_t pk = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                    pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
      pop[t] = __builtin_bit_cast(bf16x8_t, pk);
    }

    // O^T += V^T P^T : V^T operand by transpose reads of the LDS tile. Lane (lr, lq)
    // supplies the address of 4 dims of key 16 e + 4 lq + lr/4; the read returns to lane
    // lr the dim 16 dt + lr of keys 16 e + 4 lq + 0..3.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int cc = 2 * dt + ((lr & 3) >> 1);
      const int k0 = 4 * lq + (lr >> 2);
      const int k1 = 16 + k0;
      const int off0 = vlds_off(k0, cc) + 8 * (lr & 1);
      const int off1 = vlds_off(k1, cc) + 8 * (lr & 1);
      i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (i16x4_t __attribute__((address_space(3)))*)(vlds + off0));
      i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (i16x4_t __attribute__((address_space(3)))*)(vlds + off1));
      u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
      bf16x8_t vop = __builtin_bit_cast(bf16x8_t, u32x4_t{w0.x, w0.y, w1.x, w1.y});
#pragma unroll
      for (int t = 0; t < NRT; ++t)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t], o[t][dt], 0, 0, 0);
    }
  };

  // ---- main loop: two tiles in flight, chunks of at most kChunkPages pages ----
  const int chunk_keys = (int)min((int64_t)kChunkPages * S, (int64_t)1 << 30);
  Tile A, B;
  for (int c0 = j_begin; c0 < j_end; c0 += chunk_keys) {
    const int c1 = min(c0 + chunk_keys, j_end);
    stage_pages(c0, c1);
    const int nt = (c1 - c0 + kTileKeys - 1) / kTileKeys;
    load_tile(A, c0);
    int i = 0;
    for (; i + 3 <= nt; i += 2) {
      const int j0 = c0 + i * kTileKeys;
      load_tile(B, j0 + kTileKeys);
      process_tile(A, j0);
      load_tile(A, j0 + 2 * kTileKeys);
      process_tile(B, j0 + kTileKeys);
    }
    if (i + 2 == nt) {              // the last one or two tiles of the chunk
      const int j0 = c0 + i * kTileKeys;
      load_tile(B, j0 + kTileKeys);
      process_tile(A, j0);
      process_tile(B, j0 + kTileKeys);
    } else {
      process_tile(A, c0 + i * kTileKeys);
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const float l = wave_sum_rows(l_run[t]);
    if (!row_ok[t]) continue;
    const int rho = 16 * t + lr;
    const int r = rho / G;
    const int h = row_h[t];
    const int64_t row = (int64_t)(b * n + r) * a.num_q_heads + h;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? m_run[t] + __logf(l) : kNegInf;
    if (a.num_splits == 1) {
      uint16_t* op = a.out + row * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4_t v = o[t][dt] * inv;
        u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2_t*>(op + 16 * dt + 4 * lq) = w;
      }
      if (lq == 0 && a.lse != nullptr) a.lse[row] = lse;
    } else {
      float* pp = a.part_o + (row * a.num_splits + split) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4_t*>(pp + 16 * dt + 4 * lq) = o[t][dt] * inv;
      if (lq == 0) a.part_lse[row * a.num_splits + split] = lse;
    }
  }
}

// Merge of the split partials (page 2, FA4 kernel: split count from batch, heads and
// KV length): out = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - max lse), and
// lse = max + ln sum w_s. Parts with lse = -inf (no visible key) are skipped.
//
// One wave per (sequence, row, query head, 32-dim slice). Lane (stripe, c4) merges
// splits stripe, stripe + 8, ... for dims 4 c4 .. 4 c4 + 3 with a running maximum,
// issuing the loads of kCombineUnroll splits at once, so that a row's partials arrive
// in one memory round trip for up to 8 * kCombineUnroll splits; the 8 stripes are then
// merged with lane shuffles by the same rule.
constexpr int kCombineThreads = 64;
constexpr int kCombineStripes = 8;
constexpr int kCombineUnroll = 16;

__device__ __forceinline__ void merge_part(float& m, float& l, f32x4_t& acc, float m2,
                                           float l2, f32x4_t acc2) {
  const float M = fmaxf(m, m2);
  const float w1 = m == kNegInf ? 0.f : __expf(m - M);
  const float w2 = m2 == kNegInf ? 0.f : __expf(m2 - M);
  l = l * w1 + l2 * w2;
  acc = acc * w1 + acc2 * w2;
  m = M;
}

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(KernelArgs a) {
  const int lane = threadIdx.x;
  const int c4 = lane & 7;
  const int stripe = lane >> 3;
  const int64_t row = blockIdx.x / kCombineSlices;      // (b * n + r) * Hq + h
  const int slice = blockIdx.x % kCombineSlices;
  const int ns = a.num_splits;
  const float* lp = a.part_lse + row * ns;
  const float* op = a.part_o + row * ns * kHeadDim + 32 * slice + 4 * c4;

  float m = kNegInf, l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = stripe; s0 < ns; s0 += kCombineStripes * kCombineUnroll) {
    float ls[kCombineUnroll];
    f32x4_t ov[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const int s = s0 + kCombineStripes * u;
      ls[u] = s < ns ? lp[s] : kNegInf;
    }
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const int s = s0 + kCombineStripes * u;
      ov[u] = s < ns ? *reinterpret_cast<const f32x4_t*>(op + (int64_t)s * kHeadDim)
                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      if (ls[u] == kNegInf) continue;          // never touch the O of an empty part
      merge_part(m, l, acc, ls[u], 1.f, ov[u]);
    }
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    f32x4_t a2;
    a2[0] = __shfl_xor(acc[0], off);
    a2[1] = __shfl_xor(acc[1], off);
    a2[2] = __shfl_xor(acc[2], off);
    a2[3] = __shfl_xor(acc[3], off);
    merge_part(m, l, acc, m2, l2, a2);
  }
  if (stripe == 0) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const f32x4_t v = acc * inv;
    u32x2_t wv = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2_t*>(a.out + row * kHeadDim + 32 * slice + 4 * c4) = wv;
    if (slice == 0 && c4 == 0 && a.lse != nullptr)
      a.lse[row] = l > 0.f ? m + __logf(l) : kNegInf;
  }
}

int launch_split_kv(const KernelArgs& a, int row_tiles, bool fp8, void* stream) {
  dim3 grid(a.num_splits, a.num_kv_heads, a.batch);
  dim3 block(64);
  hipStream_t st = (hipStream_t)stream;
#define RATTN_LAUNCH(NRT, F8) \
  hipLaunchKernelGGL((split_kv_kernel<NRT, F8>), grid, block, 0, st, a)
  switch (row_tiles * 2 + (fp8 ? 1 : 0)) {
    case 2: RATTN_LAUNCH(1, false); break;
    case 3: RATTN_LAUNCH(1, true); break;
    case 4: RATTN_LAUNCH(2, false); break;
    case 5: RATTN_LAUNCH(2, true); break;
    case 6: RATTN_LAUNCH(3, false); break;
    case 7: RATTN_LAUNCH(3, true); break;
    case 8: RATTN_LAUNCH(4, false); break;
    case 9: RATTN_LAUNCH(4, true); break;
    default: return (int)hipErrorInvalidValue;
  }
#undef RATTN_LAUNCH
  return (int)hipGetLastError();
}

int split_kv_blocks_per_cu(int row_tiles, bool fp8) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
#define RATTN_OCC(NRT, F8) \
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, split_kv_kernel<NRT, F8>, 64, 0)
  switch (row_tiles * 2 + (fp8 ? 1 : 0)) {
    case 2: RATTN_OCC(1, false); break;
    case 3: RATTN_OCC(1, true); break;
    case 4: RATTN_OCC(2, false); break;
    case 5: RATTN_OCC(2, true); break;
    case 6: RATTN_OCC(3, false); break;
    case 7: RATTN_OCC(3, true); break;
    case 8: RATTN_OCC(4, false); break;
    case 9: RATTN_OCC(4, true); break;
    default: return 0;
  }
#undef RATTN_OCC
  return e == hipSuccess ? nb : 0;
}

int launch_combine(const KernelArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.batch * a.n * a.num_q_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(rows * kCombineSlices)),
                     dim3(kCombineThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rattn
