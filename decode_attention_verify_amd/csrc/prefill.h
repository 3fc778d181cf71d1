// Chunked prefill: attention of a chunk of many query rows per sequence (its last n
// positions, causal among themselves) over the paged cache, with the relative-position
// bias. Page 3 ("vLLM supports Reflection Beam", section on coding agents speeding up
// the implementation) times a prefill of 8 chunks of 2048 tokens at about 100K
// context; the arithmetic is the decode/verify arithmetic with n in the thousands
// (page 2, "vLLM TML Inkling support", model architecture section: a learned relative
// term added to the logits before the softmax).
//
// With thousands of rows per (sequence, KV head) the work is a dense contraction, so
// this kernel is built around the MFMA units rather than around streaming (a bf16
// cache; prefill_e4m3.h serves the E4M3 cache):
//  * one work-group of NW = 8 waves per (sequence, KV head, block of M query tokens); a
//    wave takes 16 consecutive tokens for HW query heads of the group, one 16-row MFMA
//    tile per head (3 heads for a 6-head group, 2 for 4- and 8-head groups), so
//    M = 16 * NW / (G / HW); its queries stay in registers as the B operands of
//    S^T = K Q^T;
//  * ping-pong: waves w and w + 4 share a SIMD. Each wave alternates a half of matrix
//    instructions only (P V of the previous tile, then S^T of the current one) and a
//    half of VALU work (softmax and exponentials, then its share of the next tile's
//    loads and LDS stores), and waves 4-7 run half a period behind waves 0-3, so that
//    one wave of each SIMD issues MFMAs while the other issues VALU instructions. On
//    MI355X a wave of matrix instructions and a wave of VALU instructions on one SIMD
//    run nearly as fast as each alone, while one wave mixing both gets no overlap; two
//    waves of one SIMD in the same phase (one barrier per tile) left the matrix units
//    idle while both ran their softmax;
//  * 32-key K/V tiles double-buffered in LDS in padded rows (so that every fragment
//    read's offset is an immediate), each thread loading 16 bytes of a K row and 16 of a
//    V row (16 lanes read a 256-byte row, through the caches, which the unit's other
//    blocks hit); every K or V^T fragment read from LDS feeds the MFMAs of all HW heads;
//    the page ids of a tile's loads are read from LDS a half ahead of the loads; with
//    two heads per wave a thread holds two sets of these shares, loaded two tiles
//    before they are stored (one tile with three heads, whose registers are full);
//  * the bias is sheared: for a tile at key j0, head h needs distances p0 - j0 - 31 ..
//    p0 + M - 1 - j0 (p0 the position of the block's first token), one contiguous slice
//    of M + 31 entries which the work-group stages in LDS (divided by the softmax
//    scale, in reverse order) next to the tile; row t reads key j at slice position
//    (t - t0) - (j - j0) + 31, as the initial value of its S^T accumulator, so that the
//    MFMAs leave s / scale;
//  * logits in base 2 (s / scale times scale log2 e, one FMA that also subtracts the
//    row's reference point before the exponential), masks (causal and window, compiled
//    only into the instance for tiles that cross the diagonal or the window edge), lazy
//    online softmax (one rescale test per tile for all heads, on each lane's own
//    maximum); S^T = K Q^T leaves lane (lr, lq) row lr with keys 4 lq + i, which is the
//    B operand of O^T += V^T P^T, and V^T is read back with ds_read_b64_tr_b16;
//  * work-groups are numbered so that the token blocks of one (sequence, KV head) run
//    back to back on one XCD (work-group w runs on XCD w mod 8): they stream the same
//    K/V at about the same time and share that XCD's L2.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"
#include "device_common.h"

namespace rattn {

template <int HW, int HG, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_kernel(KernelArgs a) {
  constexpr int NT = 64 * NW;                // threads
  constexpr int TB = NW / HG;                // 16-token blocks per work-group
  constexpr int M = 16 * TB;                 // query tokens per work-group
  constexpr int G = HW * HG;                 // query heads per KV head
  constexpr int SL = M + kTileKeys - 1;      // bias slice per head and tile
  constexpr int BIAS_ELEMS = G * SL;
  constexpr int BIAS_PER_THREAD = (BIAS_ELEMS + NT - 1) / NT;
  constexpr int KPP = NT / 16;               // keys one load pass of the group covers
  constexpr int SPK = kTileKeys / KPP;       // passes per K (or V) tile
  static_assert(TB * HG == NW && TB >= 1 && SPK >= 1 && SPK * KPP == kTileKeys, "shape");
  // K rows padded to 272 bytes: the four fragments of a row tile lie at fixed offsets
  // from one lane address, so that each read's offset is an immediate. On MI355X this
  // 16-byte read pattern has some bank conflicts at 272-byte rows (0.12 cycles per read
  // in a standalone probe) and none at 288, yet the 8 x 2048 prefill ran 2.5 % faster
  // at 272 (41.8 against 42.8 ms).
  constexpr int KROW = 272;
  __shared__ __attribute__((aligned(16))) unsigned char klds[2][kTileKeys * KROW];
  // V rows padded to 288 bytes: the four keys one 16-lane group of a transposing read
  // touches start 8 banks apart, and the dim offset 32 dt of each read is an immediate
  constexpr int VROW = 288;
  __shared__ __attribute__((aligned(16))) unsigned char vlds[2][kTileKeys * VROW];
  __shared__ float bias_lds[2][BIAS_ELEMS];
  __shared__ int pages_lds[2][kChunkPages + 1];   // two chunks of page ids

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
  const float inv_scale = 1.f / a.softmax_scale;
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
  const int L = __builtin_amdgcn_readfirstlane(sg.L);     // uniform (the tile loop is scalar)
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
  // the queries of the wave's rows and heads in registers, as the B operands of S^T = K Q^T
  bf16x8_t qreg[HW][4];
#pragma unroll
  for (int i = 0; i < HW; ++i) {
    const int h = g * G + hg * HW + i;
    const int64_t qr = (int64_t)b * n + (row_ok ? t_row : t0);
    const uint16_t* qrow = a.q + (qr * a.num_q_heads + h) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t v = row_ok ? ld16(qrow + 32 * s + 8 * lq) : u32x4_t{0, 0, 0, 0};
      qreg[i][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- the schedule. Group A (waves 0-3) and group B (waves 4-7) hold one wave on each
  // SIMD. A wave alternates an M half (P V of tile t - 1, then S^T of tile t: matrix
  // instructions only) and a V half (logits, softmax and exponentials of tile t, then its
  // share of the LDS stores and the next loads: VALU and memory instructions), and group
  // B runs half a period behind group A: each SIMD holds one wave in its M half and one
  // in its V half. (On MI355X a wave issuing only matrix instructions and a wave issuing
  // only VALU instructions on one SIMD each run nearly as fast as alone, while a wave
  // that mixes them gets no overlap.) A barrier ends every half: A's M(t) shares a half
  // with B's V(t - 1), A's V(t) with B's M(t).
  //
  // LDS lifetimes (half h lies between barriers h - 1 and h; A's M(t) is in half 2t + 1,
  // A's V(t) in 2t + 2, B's M(t) in 2t + 2, B's V(t) in 2t + 3):
  //  * K_t and the bias slice of tile t (buffers t & 1) are read in halves 2t + 1 and
  //    2t + 2 (the M(t) halves); V_t (buffer t & 1) in 2t + 3 and 2t + 4 (the M(t + 1)
  //    halves);
  //  * so in its V(t) a wave of group g stores its shares of K_{t+1+g}, of the bias
  //    slice of tile t + 1 + g and of V_{t+g}: each buffer is written after its
  //    previous tile's last read and before its tile's first read.
  static_assert(NW == 8, "two groups of one wave per SIMD");
  // Tiles between a share's loads and its stores. With two heads per wave the registers
  // hold two sets of shares, so a V half loads the shares it stores two tiles later
  // (about three halves of latency cover instead of one and a half); three heads per
  // wave keep one set.
  constexpr int LEAD = HW <= 2 ? 2 : 1;
  static_assert(SPK == 1, "one K and one V load per thread and tile");
  const int grp = wave >> 2;
  const int nt = (j_end - j_begin + kTileKeys - 1) / kTileKeys;   // tiles, >= 1
  const int chunk_keys = (int)min((int64_t)kChunkPages * S, (int64_t)1 << 30);   // a power of 2
  const int chunk_shift = __builtin_ctz(chunk_keys);
  const int chunk_tiles = chunk_keys / kTileKeys;                // >= 16, a power of 2

  // ---- page ids, staged in LDS per chunk of keys, two chunk buffers. The ids of chunk
  // c + 1 are staged in the V half of the chunk's first tile (group A's half 2 c T + 2,
  // B's 2 c T + 3, T tiles per chunk). The ids are read in the M half that precedes a
  // tile's loads (tile_base), LEAD tiles before its stores: the first read of chunk c + 1
  // comes at least 2 T - 5 - 2 LEAD halves after its staging began, and the last read
  // of chunk c - 1 (the buffer's previous chunk) at least 4 halves before it. ----
  const int32_t* pt_row = a.page_table + (int64_t)b * a.max_pages;
  auto stage_chunk = [&](int c) {
    const int c0 = j_begin + c * chunk_keys;
    const int c1 = min(c0 + chunk_keys, j_end);
    const int cp0 = c0 >> a.page_shift;
    const int np = ((c1 - 1) >> a.page_shift) - cp0 + 1;   // <= kChunkPages + 1
    for (int i = tid; i < np; i += NT) {
      int ph = pt_row[cp0 + i];
      if (ph < 0 || ph >= a.num_pages) {
        atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
        ph = min(max(ph, 0), a.num_pages - 1);
      }
      pages_lds[c & 1][i] = ph;
    }
  };
  // first token (in the cache) of the 16-key subtile kt of tile x (uniform arguments)
  // in two steps: the page id read from LDS (tile_page), then the token (tile_tok), so
  // that the read can be issued well before its value is used
  auto tile_js = [&](int x, int kt) {
    return min(max(j_begin + x * kTileKeys + 16 * kt, sub_lo), sub_hi);
  };
  auto tile_page = [&](int x, int kt) -> int {
    const int js = tile_js(x, kt);
    const int c = (js - j_begin) >> chunk_shift;
    const int idx = min(max((js >> a.page_shift) - ((j_begin + (c << chunk_shift)) >> a.page_shift), 0),
                        kChunkPages);
    return pages_lds[c & 1][idx];
  };
  auto tile_tok = [&](int x, int kt, int page) -> int64_t {
    const int ph = __builtin_amdgcn_readfirstlane(page);
    const int js = tile_js(x, kt);
    return ((int64_t)ph * Hkv + g) * S + (js & (S - 1));
  };

  // ---- a wave's shares of the tiles it stores in V(p): loaded in V(p - 1). Tile
  // indices outside [0, nt) load tile 0 or nt - 1 again (every load is issued) and are
  // not stored. ----
  struct Shares {
    u32x4_t k, v;                            // 16 bytes of a K row and of a V row
    float bs[BIAS_PER_THREAD];               // bias slice elements
  };
  const unsigned char* kc = (const unsigned char*)a.k_cache;
  const unsigned char* vc = (const unsigned char*)a.v_cache;
  const int ld_key = tid >> 4;               // key of the tile (wave w: 4 w .. 4 w + 3)
  const int ld_ch = tid & 15;                // 16-byte chunk of the key row
  const unsigned ld_off = (ld_key & 15) * 256 + 16 * ld_ch;   // bytes from the subtile's row 0
  auto clamp_tile = [&](int x) { return min(max(x, 0), nt - 1); };
  // this thread's bias slice elements e = tid + NT q: position e % SL of head e / SL
  // (table row bs_row, -1: no element)
  int bs_pos[BIAS_PER_THREAD], bs_row[BIAS_PER_THREAD];
#pragma unroll
  for (int q = 0; q < BIAS_PER_THREAD; ++q) {
    const int e = tid + NT * q;
    const int hi = e / SL;
    bs_pos[q] = e - hi * SL;
    bs_row[q] = e < BIAS_ELEMS ? (g * G + hi) * (a.dmax + 1) : -1;
  }
  // the byte offsets, in the caches, of the 16-key subtiles that load_shares(X, p) reads
  // (uniform), worked out a half ahead of the loads: the M half issues the two page-id
  // reads before its fragment reads and finishes the offsets after its last matrix
  // instruction, so that neither the reads' latency nor the scalar products delay the
  // V half's loads
  struct TilePages {
    int k, v;
  };
  struct TileBase {
    int64_t k, v;
  };
  // wave w reads keys 4 w .. 4 w + 3: subtile grp
  auto tile_pages = [&](int p) -> TilePages {
    return TilePages{tile_page(clamp_tile(p + 1 + grp), grp), tile_page(clamp_tile(p + grp), grp)};
  };
  auto tile_base = [&](int p, const TilePages& pg) -> TileBase {
    return TileBase{tile_tok(clamp_tile(p + 1 + grp), grp, pg.k) * 256,
                    tile_tok(clamp_tile(p + grp), grp, pg.v) * 256};
  };
  auto load_shares = [&](Shares& X, int p, const TileBase& tb) {
    const int xb = clamp_tile(p + 1 + grp);
    X.k = ld16(kc + tb.k + ld_off);
    X.v = ld16(vc + tb.v + ld_off);
    // slice element e: head e / SL of the group, distance p0 - j0 - 31 + e % SL, clamped
    // to [0, Dmax] (a masked key reads an in-range entry)
    const int d0 = p0 - (j_begin + xb * kTileKeys) - (kTileKeys - 1);
#pragma unroll
    for (int q = 0; q < BIAS_PER_THREAD; ++q) {
      const int d = min(max(d0 + bs_pos[q], 0), a.dmax);
      X.bs[q] = a.bias[bs_row[q] >= 0 ? (unsigned)(bs_row[q] + d) : 0u];
    }
  };
  // the shares into LDS (V of keys outside [k_lo, L) as zero, so that P = 0 times a stale
  // or NaN value cannot reach the accumulator)
  auto store_shares = [&](const Shares& X, int p) {
    const int xk = p + 1 + grp, xv = p + grp;
    if (xk >= 0 && xk < nt) {
      *reinterpret_cast<u32x4_t*>(klds[xk & 1] + ld_key * KROW + 16 * ld_ch) = X.k;
      // the bias divided by the softmax scale: the S accumulators' initial value. Each
      // head's slice is stored in reverse, position pos at SL - 1 - pos, so that the four
      // entries a lane's accumulator takes are ascending in LDS
#pragma unroll
      for (int q = 0; q < BIAS_PER_THREAD; ++q) {
        const int e = tid + NT * q;
        if (e < BIAS_ELEMS) bias_lds[xk & 1][e + SL - 1 - 2 * bs_pos[q]] = X.bs[q] * inv_scale;
      }
    }
    if (xv >= 0 && xv < nt) {
      u32x4_t v = X.v;
      const int j = j_begin + xv * kTileKeys + ld_key;
      if (j < k_lo || j >= L) v = u32x4_t{0, 0, 0, 0};
      *reinterpret_cast<u32x4_t*>(vlds[xv & 1] + ld_key * VROW + 16 * ld_ch) = v;
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
  // (stored reversed: key 4 lq + c of subtile kt of head i at bias_rev0 + i SL + 16 kt + c)
  const int bias_rev0 = (hg * HW) * SL + (SL - 1) - (16 * tb + lr - 4 * lq + (kTileKeys - 1));
  // tile x has a key that one of the wave's rows sees (tiles run in key order: after
  // the first tile past the wave's last row, none has)
  auto live = [&](int x) { return wave_live && j_begin + x * kTileKeys <= wave_last_p; };

  f32x4_t sacc[HW][2];                       // S^T of the current tile, M(t) -> V(t)
  bf16x8_t pop[HW];                          // P of the current tile, V(t) -> M(t + 1)

  // M(t): P V of tile t - 1, then S^T = K Q^T of tile t; each K or V^T fragment read
  // from LDS feeds the MFMAs of all HW heads
  TileBase next_base;                        // load_shares(X, t + 1) of V(t), from M(t)
  auto m_half = [&](int t) {
    const TilePages next_pages = tile_pages(t + LEAD);
    if (t >= 1 && live(t - 1)) {
      const unsigned char* vl = vlds[(t - 1) & 1];
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
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, u32x4_t{w0.x, w0.y, w1.x, w1.y});
#pragma unroll
        for (int i = 0; i < HW; ++i) {
          o[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[i], o[i][dt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t < nt && live(t)) {
      const unsigned char* kl = klds[t & 1];
      const float* bl = bias_lds[t & 1];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < HW; ++i) {
          // the accumulators start at bias / scale, so that they end at s / scale (the
          // logit of key 4 lq + c of subtile kt for the lane's row, before the scale)
          const int bp = bias_rev0 + i * SL + 16 * kt;
          sacc[i][kt] = f32x4_t{bl[bp], bl[bp + 1], bl[bp + 2], bl[bp + 3]};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t kop = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(kl + (16 * kt + lr) * KROW + 16 * (4 * s + lq)));
#pragma unroll
          for (int i = 0; i < HW; ++i) {
            sacc[i][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[i][s], sacc[i][kt], 0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    next_base = tile_base(t + LEAD, next_pages);
  };

  // V(t): masks (FAST = false: the tiles that cross the diagonal or the window edge),
  // the tile maximum, the rare rescale, P = exp(s - m); then the wave's share of the
  // stores and the next loads
  // X0: the shares this V half stores; X1 (LEAD = 2): the next V half's
  Shares X0, X1;
  auto v_half = [&](int t, auto fast_tag, Shares& X) {
    constexpr bool FAST = decltype(fast_tag)::value;
    if (live(t)) {
      const int j0 = j_begin + t * kTileKeys;
      (void)j0;
      // sv = s / scale (masked keys: -inf) and each lane's maximum of each head in base 2
      float sv[HW][2][4];
      float lm[HW];
      bool grow_any = false;
#pragma unroll
      for (int i = 0; i < HW; ++i) {
        float x = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float sc = sacc[i][kt][c];
            if (!FAST) {
              const int dist = row_p - (j0 + 16 * kt + 4 * lq + c);
              const bool vis = row_ok && dist >= 0 && (W == 0 || dist < W);
              sc = vis ? sc : kNegInf;
            }
            sv[i][kt][c] = sc;
            x = fmaxf(x, sc);
          }
        lm[i] = x * scale2;
        // the reference point m of a row moves only when its tile maximum passes m by
        // kRescaleSlack2: the test on each lane's own maximum is the same test
        grow_any |= lm[i] > m_run[i] + kRescaleSlack2;
      }
      // one test for all heads, the rare rescale in one branch (the row maximum from
      // the 4 lanes of each row)
      if (__ballot(grow_any) != 0) {
#pragma unroll
        for (int i = 0; i < HW; ++i) {
          const float mt = wave_max_rows(lm[i]);
          const bool grow = mt > m_run[i] + kRescaleSlack2;
          const float m_new = grow ? mt : m_run[i];
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[i] - m_new) : 1.f;
          l_run[i] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[i][dt] *= alpha;
          m_run[i] = m_new;
        }
      }
      // P = exp2(sv scale log2 e - m), packed as the B operand of O^T += V^T P^T
#pragma unroll
      for (int i = 0; i < HW; ++i) {
        const float mb = -(m_run[i] == kNegInf ? 0.f : m_run[i]);
        float pv[2][4];
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i][kt][c], scale2, mb));
            psum += p;
            pv[kt][c] = p;
          }
        l_run[i] += psum;
        const u32x4_t pk = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                            pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
        pop[i] = __builtin_bit_cast(bf16x8_t, pk);
      }
    }
    store_shares(X, t);
    if ((t & (chunk_tiles - 1)) == 0 && t + chunk_tiles < nt)
      stage_chunk((t >> (chunk_shift - 5)) + 1);             // chunk_tiles = 2^(chunk_shift - 5)
    load_shares(X, t + LEAD, next_base);
  };

  // ---- prologue: chunk 0's page ids; group A stores what its V(-1) would, group B
  // what its V(-2) would, then B's V(-1) shares A's M(0) half. Each group ends holding
  // the shares of V(0) (and of V(1) with two sets). ----
  auto load_at = [&](Shares& X, int p) { load_shares(X, p, tile_base(p, tile_pages(p))); };
  stage_chunk(0);
  __syncthreads();
  load_at(X0, grp ? -2 : -1);
  store_shares(X0, grp ? -2 : -1);
  if constexpr (LEAD == 2) {
    if (grp) {
      load_at(X0, -1);
      __syncthreads();
      store_shares(X0, -1);
    }
    load_at(X0, 0);
    load_at(X1, 1);
    __syncthreads();
  } else {
    load_at(X0, grp ? -1 : 0);
    __syncthreads();
    if (grp) {
      store_shares(X0, -1);
      load_at(X0, 0);
      __syncthreads();
    }
  }

  // ---- tile loop: fast tiles (every key visible to every row: no mask code) form one
  // contiguous run; the masked tiles before it (window edge) and after it (diagonal)
  // run in loops of their own, so that each loop body holds one instance of the
  // softmax. Fast tiles: j0 + 31 <= p0, and with a window p_last - j0 <= W - 1. ----
  int x_lo = 0;
  if (W > 0) {
    const int first = p_last - W + 1 - j_begin;          // smallest fast j0 - j_begin
    x_lo = first <= 0 ? 0 : min((first + kTileKeys - 1) / kTileKeys, nt);
  }
  const int last = p0 - (kTileKeys - 1) - j_begin;        // largest fast j0 - j_begin
  const int x_hi = last < 0 ? x_lo : max(x_lo, min(last / kTileKeys + 1, nt));
  int t = 0;
  // tiles t .. t_end - 1; with two sets, V(t) stores X0 and V(t + 1) X1, and a run of
  // odd length leaves the sets exchanged for the next run
  auto run = [&](int t_end, auto fast_tag) {
    for (; t + 1 < t_end; t += 2) {
      m_half(t);
      __syncthreads();
      v_half(t, fast_tag, X0);
      __syncthreads();
      m_half(t + 1);
      __syncthreads();
      v_half(t + 1, fast_tag, X1);
      __syncthreads();
    }
    if (t < t_end) {
      m_half(t);
      __syncthreads();
      v_half(t, fast_tag, X0);
      __syncthreads();
      ++t;
      const Shares x = X0;
      X0 = X1;
      X1 = x;
    }
  };
  // (one set keeps loops of its own: written as runs of two steps, the same schedule
  // compiled to a three-head kernel with more registers and a slower loop)
  if constexpr (LEAD == 2) {
    run(x_lo, std::false_type{});
    run(x_hi, std::true_type{});
    run(nt, std::false_type{});
  } else {
    for (; t < x_lo; ++t) {
      m_half(t);
      __syncthreads();
      v_half(t, std::false_type{}, X0);
      __syncthreads();
    }
    for (; t < x_hi; ++t) {
      m_half(t);
      __syncthreads();
      v_half(t, std::true_type{}, X0);
      __syncthreads();
    }
    for (; t < nt; ++t) {
      m_half(t);
      __syncthreads();
      v_half(t, std::false_type{}, X0);
      __syncthreads();
    }
  }
  m_half(nt);                                 // P V of the last tile
  if (!grp) __syncthreads();                  // pairs with group B's last barrier

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
