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
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
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

__device__ __forceinline__ float wave_max_rows(float x) {
  // max over the 4 lanes lr, lr+16, lr+32, lr+48 that hold the same query row
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
__device__ __forceinline__ int vlds_off(int k, int cc) {
  return k * 256 + ((cc ^ ((k & 7) << 1)) << 4);
}

template <int NRT, bool FP8>
__global__ __launch_bounds__(64) void split_kv_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char vlds[kTileKeys * 256];

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
  if (j_begin >= L) return;                  // empty split: the combine skips it
  const int j_end = min(j_begin + a.keys_per_split, L);
  const int ntiles = (j_end - j_begin + kTileKeys - 1) / kTileKeys;
  // tiles at or after `fast_lo` and before `fast_hi` need no mask: every key is
  // visible to every row at a distance in [0, W-1]
  const int fast_lo = W > 0 ? max(0, L - W) : 0;
  const int fast_hi = L - n - (kTileKeys - 1);   // j0 <= fast_hi

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
      // the d-permutation must match the K operand: bf16 K gives each lane 8 dims at
      // 32 s + 8 lq; an E4M3 K row gives 16 dims at 64 (s/2) + 16 lq
      const int d0 = FP8 ? 64 * (s >> 1) + 16 * lq + 8 * (s & 1) : 32 * s + 8 * lq;
      u32x4_t v = row_ok[t] ? ld16(qrow + d0) : u32x4_t{0, 0, 0, 0};
      qreg[t][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const float* brow[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) brow[t] = a.bias + (int64_t)row_h[t] * (a.dmax + 1);

  // ---- page ids: one vector of up to 64 consecutive page-table entries ----
  const int32_t* pt_row = a.page_table + (int64_t)b * a.max_pages;
  const int last_page = (L - 1) >> a.page_shift;
  int pt_first = j_begin >> a.page_shift;
  int pt_vec = 0;
  {
    const int pi = pt_first + lane;
    pt_vec = pi <= last_page ? pt_row[pi] : 0;
  }
  auto phys_of = [&](int pidx) -> int {
    if (pidx - pt_first >= 64) {               // uniform: refresh the window of ids
      pt_first = pidx;
      const int pi = pt_first + lane;
      pt_vec = pi <= last_page ? pt_row[pi] : 0;
    }
    int ph = __builtin_amdgcn_readlane(pt_vec, pidx - pt_first);
    if (ph < 0 || ph >= a.num_pages) {
      if (lane == 0) atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
      ph = min(max(ph, 0), a.num_pages - 1);
    }
    return ph;
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
  auto load_tile = [&](Tile& T, int j0) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int jt = j0 + 16 * kt;
      const bool valid = (jt < L) && (jt + 16 > k_lo);      // uniform
      if (valid) {
        const int ph = phys_of(jt >> a.page_shift);
        const int64_t tok0 = ((int64_t)ph * Hkv + g) * S + (jt & (S - 1));
        if (!FP8) {
          const unsigned char* kp =
              (const unsigned char*)a.k_cache + (tok0 + lr) * 256 + 16 * lq;
#pragma unroll
          for (int s = 0; s < 4; ++s) T.k[kt][s] = ld16(kp + 64 * s);
#pragma unroll
          for (int u = 0; u < 4; ++u) {   // V keys 4u + lq of this subtile, chunk lr
            const unsigned char* vp = (const unsigned char*)a.v_cache +
                                      (tok0 + 4 * u + lq) * 256 + 16 * lr;
            T.v[4 * kt + u] = ld16(vp);
          }
        } else {
          const unsigned char* kp =
              (const unsigned char*)a.k_cache + (tok0 + lr) * 128 + 16 * lq;
          T.k[kt][0] = ld16(kp);
          T.k[kt][1] = ld16(kp + 64);
#pragma unroll
          for (int u = 0; u < 2; ++u) {   // V keys 8u + lane/8 of this subtile, chunk lane%8
            const unsigned char* vp = (const unsigned char*)a.v_cache +
                                      (tok0 + 8 * u + (lane >> 3)) * 128 + 16 * (lane & 7);
            T.v[2 * kt + u] = ld16(vp);
          }
          T.ks[kt] = *reinterpret_cast<const f32x4_t*>(a.k_scale + tok0 + 4 * lq);
          T.vs[kt] = *reinterpret_cast<const f32x4_t*>(a.v_scale + tok0 + 4 * lq);
        }
      } else {
#pragma unroll
        for (int s = 0; s < KV_REGS; ++s) T.k[kt][s] = u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < V_LOADS / 2; ++u) T.v[(V_LOADS / 2) * kt + u] = u32x4_t{0, 0, 0, 0};
        if (FP8) {
          T.ks[kt] = f32x4_t{0, 0, 0, 0};
          T.vs[kt] = f32x4_t{0, 0, 0, 0};
        }
      }
      // bias: row r of head h reads B[h][p_r - j] for its 4 keys; rows of one head are
      // the same slice shifted by their offset r (the sheared access)
#pragma unroll
      for (int t = 0; t < NRT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int dist = row_p[t] - (jt + 4 * lq + i);
          dist = min(max(dist, 0), a.dmax);
          T.bias[t][kt][i] = (row_ok[t] && valid) ? brow[t][dist] : 0.f;
        }
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

    // S^T = K Q^T : lane holds row lr (+16 t), keys 4 lq + i of each 16-key subtile
    bf16x8_t kop[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (!FP8) {
#pragma unroll
        for (int s = 0; s < 4; ++s) kop[kt][s] = __builtin_bit_cast(bf16x8_t, T.k[kt][s]);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x2_t c0 = e4m3x4_to_bf16x4(T.k[kt][u].x), c1 = e4m3x4_to_bf16x4(T.k[kt][u].y);
          u32x2_t c2 = e4m3x4_to_bf16x4(T.k[kt][u].z), c3 = e4m3x4_to_bf16x4(T.k[kt][u].w);
          kop[kt][2 * u] = __builtin_bit_cast(bf16x8_t, u32x4_t{c0.x, c0.y, c1.x, c1.y});
          kop[kt][2 * u + 1] = __builtin_bit_cast(bf16x8_t, u32x4_t{c2.x, c2.y, c3.x, c3.y});
        }
      }
    }
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
      const float m_new = fmaxf(m_run[t], mt);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float mb = -m_use * kLog2e;
      const float alpha = __builtin_amdgcn_exp2f(__builtin_fmaf(m_run[t], kLog2e, mb));
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
      l_run[t] = __builtin_fmaf(l_run[t], alpha, psum);
      m_run[t] = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
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

  // ---- main loop, two tiles in flight ----
  Tile A, B;
  load_tile(A, j_begin);
  int i = 0;
  for (; i + 2 <= ntiles; i += 2) {
    const int j0 = j_begin + i * kTileKeys;
    load_tile(B, j0 + kTileKeys);
    process_tile(A, j0);
    if (i + 2 < ntiles) load_tile(A, j0 + 2 * kTileKeys);
    process_tile(B, j0 + kTileKeys);
  }
  if (i < ntiles) process_tile(A, j_begin + i * kTileKeys);

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
// lse = max + ln sum w_s. One 256-thread work-group per (sequence, row, query head).
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(KernelArgs a) {
  __shared__ float w_s[kMaxSplits];
  __shared__ float red[kCombineThreads / 64];
  __shared__ f32x2_t acc_s[kCombineThreads / 64][64];
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  const int lane = tid & 63;
  const int64_t row = blockIdx.x;                  // (b * n + r) * Hq + h
  const int b = (int)(row / ((int64_t)a.n * a.num_q_heads));
  const int n = a.n;
  int L = a.seq_lens[b];
  L = min(max(L, n), a.max_seq_len);
  const int W = a.window;
  const int k_lo = W > 0 ? max(0, L - n + 1 - W) : 0;
  const int base = k_lo & ~(kTileKeys - 1);
  const int ns = min(a.num_splits, (L - base + a.keys_per_split - 1) / a.keys_per_split);
  const float* lp = a.part_lse + row * a.num_splits;
  const float* op = a.part_o + row * a.num_splits * kHeadDim;

  float m = kNegInf;
  for (int s = tid; s < ns; s += kCombineThreads) m = fmaxf(m, lp[s]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wid] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();

  float den = 0.f;
  for (int s = tid; s < ns; s += kCombineThreads) {
    const float ls = lp[s];
    const float w = ls == kNegInf ? 0.f : __expf(ls - m);
    w_s[s] = w;
    den += w;
  }
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  if (lane == 0) red[wid] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) den += red[w];

  f32x2_t acc = {0.f, 0.f};
  for (int s = wid; s < ns; s += kCombineThreads / 64) {
    const float w = w_s[s];
    if (w != 0.f) {
      const f32x2_t v = *reinterpret_cast<const f32x2_t*>(op + (int64_t)s * kHeadDim + 2 * lane);
      acc += w * v;
    }
  }
  acc_s[wid][lane] = acc;
  __syncthreads();
  if (wid == 0) {
    f32x2_t t = acc_s[0][lane];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) t += acc_s[w][lane];
    const float inv = den > 0.f ? 1.f / den : 0.f;
    *reinterpret_cast<unsigned int*>(a.out + row * kHeadDim + 2 * lane) =
        pack_bf16x2(t.x * inv, t.y * inv);
    if (lane == 0 && a.lse != nullptr) a.lse[row] = m + __logf(den);
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

int launch_combine(const KernelArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.batch * a.n * a.num_q_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)rows), dim3(kCombineThreads), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rattn
