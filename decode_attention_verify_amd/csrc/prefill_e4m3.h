// Chunked prefill over an E4M3 cache: attention of a chunk of many query rows per
// sequence (its last n positions, causal among themselves) over the paged cache, with
// the relative-position bias. Page 3 ("vLLM supports Reflection Beam", section on coding
// agents speeding up the implementation) times a prefill of 8 chunks of 2048 tokens at
// about 100K context; page 2's roadmap and page 3's support section name an FP8 KV
// cache. The arithmetic is the decode/verify arithmetic with n in the thousands (page
// 2, "vLLM TML Inkling support", model architecture section: a learned relative term
// added to the logits before the softmax).
//
// The layout of prefill.h (a bf16 cache), with its waves in step instead of in
// ping-pong: here each tile's decode, scales and second P V product make the VALU work
// of a tile larger than its matrix work, and two waves of a SIMD sharing the VALU in the
// same phase ran faster than one wave at a time (8 chunks of 2048 at 100K on MI355X:
// 65.0 ms against 73.7 ms in ping-pong):
//  * one work-group of NW = 8 waves (two per SIMD) per (sequence, KV head, block of M
//    query tokens); a wave takes 16 consecutive tokens for HW query heads of the group,
//    one 16-row MFMA tile per head, so M = 16 * NW / (G / HW);
//  * each wave's queries sit in LDS in MFMA operand order (one 16-byte read per lane and
//    head per k-step), which leaves the registers to the O accumulators;
//  * a 32-key tile of K and V codes takes one 16-byte load per thread (8 lanes per
//    128-byte key row); the codes are decoded exactly to bf16 on their way into LDS;
//    the tile's 32 K and 32 V scales are staged in LDS beside it; the next tile's loads
//    are in flight while a tile is attended; tiles are double-buffered in LDS with one
//    barrier per tile; every K or V fragment read from LDS feeds the MFMAs of all HW
//    heads;
//  * the bias is sheared as in prefill.h and staged in LDS, times log2 e;
//  * the K scale multiplies each logit column (with the softmax scale) before the bias
//    is added; the V scale multiplies each P column, and P times the V scale, which is
//    not a bf16 value, goes to the matrix units as two bf16 parts: the rounded value and
//    its rounding remainder, in a second P V product (the row sums take P unscaled);
//  * masks (causal and window, compiled only into the instance for tiles that cross the
//    diagonal or the window edge), lazy online softmax (one rescale test per tile for
//    all heads); logits in base 2, held in registers from the tile maximum to the
//    exponentials; each head's P V MFMAs follow its exponentials, so that the next
//    head's VALU work overlaps them;
//  * work-groups are numbered so that the token blocks of one (sequence, KV head) run
//    back to back on one XCD (work-group w runs on XCD w mod 8).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"
#include "device_common.h"

namespace rattn {

template <int HW, int HG, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_e4m3_kernel(KernelArgs a) {
  constexpr int NT = 64 * NW;                // threads
  constexpr int TB = NW / HG;                // 16-token blocks per work-group
  constexpr int M = 16 * TB;                 // query tokens per work-group
  constexpr int G = HW * HG;                 // query heads per KV head
  constexpr int SL = M + kTileKeys - 1;      // bias slice per head and tile
  constexpr int BIAS_ELEMS = G * SL;
  constexpr int BIAS_PER_THREAD = (BIAS_ELEMS + NT - 1) / NT;
  static_assert(TB * HG == NW && TB >= 1, "shape");
  // 32 keys x 128 bytes of K, then of V, one 16-byte load per thread
  static_assert(NT == 2 * kTileKeys * 8, "one E4M3 load per thread per tile");
  // decoded tiles with padded rows (K 272 bytes, V 288), as in the bf16 prefill kernel:
  // every fragment read's offset from one lane address is an immediate
  constexpr int KROW = 272, VROW = 288;
  __shared__ __attribute__((aligned(16))) unsigned char klds[2][kTileKeys * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char vlds[2][kTileKeys * VROW];
  __shared__ float bias_lds[2][BIAS_ELEMS];
  __shared__ int pages_lds[kChunkPages + 1];
  // a tile's 32 K scales, then its 32 V scales
  __shared__ __attribute__((aligned(16))) float scale_lds[2][64];
  // each wave's queries in MFMA operand order: block (head i, k-step s) holds lane l's
  // 16 bytes at l * 16, read back with one 16-byte LDS read per lane
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[NW][HW][4][1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = wave % TB;                  // this wave's 16-token block
  const int hg = wave / TB;                  // this wave's share of the group's heads
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int n = a.n;
  const int64_t Hkv = a.num_kv_heads;
  const int S = a.page_size;
  const int W = a.window;
  const float scale2 = a.softmax_scale * kLog2e;
  constexpr float kRescaleSlack2 = 8.f;      // kRescaleSlack in base 2
  constexpr float kLn2 = 0.6931471805599453f;

  // ---- which (sequence, KV head, token block): consecutive logical ids on one XCD ----
  const int NB = (n + M - 1) / M;
  const int64_t total = (int64_t)a.batch * Hkv * NB;
  const int64_t per_xcd = (int64_t)gridDim.x / 8;          // the grid is a multiple of 8
  const int64_t li = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (li >= total) return;                                 // uniform over the group
  const int64_t u = li / NB;
  const int blk = (int)(li - u * NB);
  const int b = (int)(u / Hkv);
  const int g = (int)(u - (int64_t)b * Hkv);

  const SeqGeom sg = seq_geom(a, b, n, true);              // length clamped into [n, max]
  const int L = sg.L;
  const int t0 = blk * M;                                  // tokens [t0, t1) of the chunk
  const int t1 = min(t0 + M, n);
  const int p0 = L - n + t0;                               // position of token t0
  const int p_last = L - n + t1 - 1;
  const int k_lo = W > 0 ? max(0, p0 - W + 1) : 0;         // first key any row sees
  const int j_begin = k_lo & ~(kTileKeys - 1);
  const int j_end = p_last + 1;
  const int sub_lo = k_lo & ~15;
  const int sub_hi = p_last & ~15;

  // ---- this lane's row: token t_row, its position, its HW heads' queries ----
  const int t_row = t0 + 16 * tb + lr;
  const bool row_ok = t_row < t1;
  const int row_p = p0 + 16 * tb + lr;
  const int wave_last_p = p0 + min(16 * tb + 15, t1 - t0 - 1);   // last row of the wave
  const bool wave_live = 16 * tb < t1 - t0;
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const int h = g * G + hg * HW + i;
    const int64_t qr = (int64_t)b * n + (row_ok ? t_row : t0);
    const uint16_t* qrow = a.q + (qr * a.num_q_heads + h) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t v = row_ok ? ld16(qrow + 32 * s + 8 * lq) : u32x4_t{0, 0, 0, 0};
      *reinterpret_cast<u32x4_t*>(&q_lds[wave][i][s][16 * lane]) = v;
    }
  }
  // (each wave reads only its own queries, after its own writes: no barrier needed)

  // ---- page ids of a chunk of keys, staged in LDS ----
  const int32_t* pt_row = a.page_table + (int64_t)b * a.max_pages;
  int chunk_p0 = 0;
  auto stage_pages = [&](int c0, int c1) {
    __syncthreads();                         // the previous chunk's ids and tiles are done
    chunk_p0 = c0 >> a.page_shift;
    const int np = ((c1 - 1) >> a.page_shift) - chunk_p0 + 1;   // <= kChunkPages + 1
    for (int i = tid; i < np; i += NT) {
      int ph = pt_row[chunk_p0 + i];
      if (ph < 0 || ph >= a.num_pages) {
        atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
        ph = min(max(ph, 0), a.num_pages - 1);
      }
      pages_lds[i] = ph;
    }
    __syncthreads();
  };
  auto phys_at = [&](int jt) -> int {
    const int idx = min(max((jt >> a.page_shift) - chunk_p0, 0), kChunkPages);
    return __builtin_amdgcn_readfirstlane(pages_lds[idx]);
  };

  // ---- a tile's loads: slot m = (K|V, 16-key subtile); thread tid reads 16 bytes of key
  // tid / 16 of the subtile (a wave reads 4 whole key rows, 1 KiB contiguous) ----
  struct Tile {
    u32x4_t x;                               // 16 codes of a K or V row
    float sc;                                // threads 0..63: a K or V scale
    float bs[BIAS_PER_THREAD];
  };
  const unsigned char* kc = (const unsigned char*)a.k_cache;
  const unsigned char* vc = (const unsigned char*)a.v_cache;
  // thread tid reads K (tid < 256) or V, key f_key of the tile, 16 codes at f_ch
  const int f_kv = (tid >> 8) & 1;
  const int f_key = (tid >> 3) & 31;
  const int f_ch = tid & 7;
  auto load_tile = [&](Tile& X, int j0) {
    int64_t tok0[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // a subtile with no key in [k_lo, p_last] reads the nearest one that has
      const int js = min(max(j0 + 16 * kt, sub_lo), sub_hi);
      tok0[kt] = ((int64_t)phys_at(js) * Hkv + g) * S + (js & (S - 1));
    }
    const int64_t tok = (f_key >> 4 ? tok0[1] : tok0[0]) + (f_key & 15);
    X.x = ld16((f_kv ? vc : kc) + tok * kHeadDim + 16 * f_ch);   // cached: the unit's other blocks read it too
    if (tid < 64) {
      const int64_t st = (tid & 16 ? tok0[1] : tok0[0]) + (tid & 15);
      X.sc = (tid & 32 ? a.v_scale : a.k_scale)[st];
    }
#pragma unroll
    for (int q = 0; q < BIAS_PER_THREAD; ++q) {
      // slice element e: head e / SL of the group, distance p0 - j0 - 31 + e % SL,
      // clamped to [0, Dmax] (a masked key reads an in-range entry)
      const int e = tid + NT * q;
      const int hi = e / SL;
      const int d = min(max(p0 - j0 - (kTileKeys - 1) + (e - hi * SL), 0), a.dmax);
      const unsigned idx = e < BIAS_ELEMS ? (unsigned)((g * G + hi) * (a.dmax + 1) + d) : 0u;
      X.bs[q] = a.bias[idx];
    }
  };

  // ---- running state: per head, the lane's row ----
  f32x4_t o[HW][8];
  float m_run[HW], l_run[HW];
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    m_run[i] = kNegInf;
    l_run[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[i][dt] = f32x4_t{0, 0, 0, 0};
  }
  // this lane's bias slice position for key 4 lq of subtile 0, at head 0 of the wave
  const int bias_pos0 = (hg * HW) * SL + 16 * tb + lr - 4 * lq + (kTileKeys - 1);

  // the tile in registers -> LDS buffer `buf` (V of keys outside [k_lo, L) as zero, so
  // that P = 0 times a stale or NaN value cannot reach the accumulator)
  auto store_tile = [&](const Tile& X, int j0, int buf) {
    unsigned char* kl = klds[buf];
    unsigned char* vl = vlds[buf];
    float* bl = bias_lds[buf];
    const bool edge = j0 < k_lo || j0 + kTileKeys > L;
    // 16 codes -> 16 bf16 values (two 16-byte chunks of the row)
    u32x4_t raw = X.x;
    const int j = j0 + f_key;
    if (f_kv && edge && (j < k_lo || j >= L)) raw = u32x4_t{0, 0, 0, 0};
    const u32x2_t c0 = e4m3x4_to_bf16x4(raw.x), c1 = e4m3x4_to_bf16x4(raw.y);
    const u32x2_t c2 = e4m3x4_to_bf16x4(raw.z), c3 = e4m3x4_to_bf16x4(raw.w);
    const u32x4_t lo = {c0.x, c0.y, c1.x, c1.y}, hi = {c2.x, c2.y, c3.x, c3.y};
    if (f_kv) {
      *reinterpret_cast<u32x4_t*>(vl + f_key * VROW + 32 * f_ch) = lo;
      *reinterpret_cast<u32x4_t*>(vl + f_key * VROW + 32 * f_ch + 16) = hi;
    } else {
      *reinterpret_cast<u32x4_t*>(kl + f_key * KROW + 32 * f_ch) = lo;
      *reinterpret_cast<u32x4_t*>(kl + f_key * KROW + 32 * f_ch + 16) = hi;
    }
    if (tid < 64) scale_lds[buf][tid] = X.sc;
#pragma unroll
    for (int q = 0; q < BIAS_PER_THREAD; ++q) {
      const int e = tid + NT * q;
      if (e < BIAS_ELEMS) bl[e] = X.bs[q] * kLog2e;   // base-2 logits
    }
  };
  // attention of this wave's rows over the tile in LDS buffer `buf`
  auto compute_tile = [&](int j0, int buf, auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const unsigned char* kl = klds[buf];
    const unsigned char* vl = vlds[buf];
    const float* bl = bias_lds[buf];
    if (!FAST && (!wave_live || j0 > wave_last_p)) return;   // every key after every row

    // S^T = K Q^T for the HW heads; each K fragment feeds all of them. The matrix
    // instructions run at a raised wave priority, so that the SIMD's other wave, in its
    // exponentials, yields the issue slot to them (the chunked prefill at 100K: 46.5 ms
    // against 46.9)
    __builtin_amdgcn_s_setprio(1);
    f32x4_t sacc[HW][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < HW; ++i) sacc[i][kt] = f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t kop = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(kl + (16 * kt + lr) * KROW + 16 * (4 * s + lq)));
#pragma unroll
        for (int i = 0; i < HW; ++i) {
          const bf16x8_t qop = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(&q_lds[wave][i][s][16 * lane]));
          sacc[i][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop, sacc[i][kt], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
    // E4M3: the K scales of this lane's keys 4 lq + c of each subtile (times the logit
    // scale); the V scales are read where P is made
    f32x4_t ks[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      ks[kt] = *reinterpret_cast<const f32x4_t*>(&scale_lds[buf][16 * kt + 4 * lq]) * scale2;
    // logits (with masks on the tiles that need them) of head i, key (kt, c)
    // logits in base 2 (scaled by log2 e): the exponentials need no multiply
    auto logit = [&](int i, int kt, int c) {
      float sc = __builtin_fmaf(sacc[i][kt][c], ks[kt][c],
                                bl[bias_pos0 + i * SL - 16 * kt - c]);
      if (!FAST) {
        const int dist = row_p - (j0 + 16 * kt + 4 * lq + c);
        const bool vis = row_ok && dist >= 0 && (W == 0 || dist < W);
        sc = vis ? sc : kNegInf;
      }
      return sc;
    };
    // each head's tile maximum; one test for all heads, the rare rescale in one branch
    float mt[HW];
    float sv[HW][2][4];
    bool grow_any = false;
#pragma unroll
    for (int i = 0; i < HW; ++i) {
      float x = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sv[i][kt][c] = logit(i, kt, c);
          x = fmaxf(x, sv[i][kt][c]);
        }
      mt[i] = wave_max_rows(x);
      grow_any |= mt[i] > m_run[i] + kRescaleSlack2;
    }
    if (__ballot(grow_any) != 0) {
#pragma unroll
      for (int i = 0; i < HW; ++i) {
        const bool grow = mt[i] > m_run[i] + kRescaleSlack2;
        const float m_new = grow ? mt[i] : m_run[i];
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[i] - m_new) : 1.f;
        l_run[i] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[i][dt] *= alpha;
        m_run[i] = m_new;
      }
    }
    // V^T fragments of the tile (each feeds all HW heads)
    bf16x8_t vop[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int cc = 2 * dt + ((lr & 3) >> 1);
      const int k0 = 4 * lq + (lr >> 2);
      const int off0 = k0 * VROW + 16 * cc + 8 * (lr & 1);
      const int off1 = (16 + k0) * VROW + 16 * cc + 8 * (lr & 1);
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (i16x4_t __attribute__((address_space(3)))*)(const_cast<unsigned char*>(vl) + off0));
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (i16x4_t __attribute__((address_space(3)))*)(const_cast<unsigned char*>(vl) + off1));
      const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
      vop[dt] = __builtin_bit_cast(bf16x8_t, u32x4_t{w0.x, w0.y, w1.x, w1.y});
    }
    f32x4_t vs[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      vs[kt] = *reinterpret_cast<const f32x4_t*>(&scale_lds[buf][32 + 16 * kt + 4 * lq]);
    // per head: P = exp(s - m) from the logits again, packed as the B operand, then
    // O^T += V^T P^T (the next head's exponentials overlap these MFMAs)
#pragma unroll
    for (int i = 0; i < HW; ++i) {
      const float mb = -(m_run[i] == kNegInf ? 0.f : m_run[i]);
      float pv[2][4];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float p = __builtin_amdgcn_exp2f(sv[i][kt][c] + mb);
          psum += p;
          pv[kt][c] = p > 0.f ? p * vs[kt][c] : 0.f;
        }
      l_run[i] += psum;
      const u32x4_t pk = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                          pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
      const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pk);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pop, o[i][dt], 0, 0, 0);
      {
        // P times the V scales is not a bf16 value: its rounding remainder in a second
        // PV product, so that one visible key gives its value to within the output's
        // own rounding
        const u32x4_t pr = {pack_bf16x2_rem(pv[0][0], pv[0][1], pk.x),
                            pack_bf16x2_rem(pv[0][2], pv[0][3], pk.y),
                            pack_bf16x2_rem(pv[1][0], pv[1][1], pk.z),
                            pack_bf16x2_rem(pv[1][2], pv[1][3], pk.w)};
        const bf16x8_t pop_lo = __builtin_bit_cast(bf16x8_t, pr);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          o[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pop_lo, o[i][dt], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // ---- tile loop: the next tile's loads in flight while a tile is attended. Tiles
  // that need no mask form one contiguous run; the masked tiles before and after it run
  // in loops of their own, so that each loop body holds one instance of the attention.
  const int chunk_keys = (int)min((int64_t)kChunkPages * S, (int64_t)1 << 30);
  Tile R;
  for (int c0 = j_begin; c0 < j_end; c0 += chunk_keys) {
    const int c1 = min(c0 + chunk_keys, j_end);
    stage_pages(c0, c1);
    const int nt = (c1 - c0 + kTileKeys - 1) / kTileKeys;
    // fast tiles i: c0 + 32 i + 31 <= p0, and with a window p_last - (c0 + 32 i) <= W - 1
    int i_lo = 0;
    if (W > 0) {
      const int first = p_last - W + 1 - c0;             // smallest fast j0 - c0
      i_lo = first <= 0 ? 0 : min((first + kTileKeys - 1) / kTileKeys, nt);
    }
    const int last = p0 - (kTileKeys - 1) - c0;           // largest fast j0 - c0
    const int i_hi = last < 0 ? i_lo : max(i_lo, min(last / kTileKeys + 1, nt));
    load_tile(R, c0);
    auto step = [&](int i, auto fast_tag) {
      const int j0 = c0 + i * kTileKeys;
      const int buf = i & 1;
      store_tile(R, j0, buf);
      if (i + 1 < nt) load_tile(R, j0 + kTileKeys);
      __syncthreads();                       // tile i and its bias slices are in LDS
      compute_tile(j0, buf, fast_tag);
    };
    int i = 0;
    for (; i < i_lo; ++i) step(i, std::false_type{});
    for (; i < i_hi; ++i) step(i, std::true_type{});
    for (; i < nt; ++i) step(i, std::false_type{});
  }

  // ---- epilogue: every row's output and log-sum-exp, per head ----
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const float l = wave_sum_rows(l_run[i]);
    if (!row_ok) continue;
    const int h = g * G + hg * HW + i;
    const int64_t row = ((int64_t)b * n + t_row) * a.num_q_heads + h;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = a.out + row * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4_t v = o[i][dt] * inv;
      const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2_t*>(op + 16 * dt + 4 * lq) = w;
    }
    // m_run is in base 2
    if (lq == 0 && a.lse != nullptr)
      a.lse[row] = l > 0.f ? m_run[i] * kLn2 + __logf(l) : kNegInf;
  }
}

}  // namespace rattn
