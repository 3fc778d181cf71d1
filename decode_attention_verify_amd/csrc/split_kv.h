// The split kernel: the attention of one decode/verify call over a piece of the keys.
//
// Method (page 2 "vLLM TML Inkling support", model architecture section): logits
// s_j = scale * q.k_j + B[h][min(p - j, Dmax)], softmax over the visible keys. Page 1
// ("vLLM supports Inkling 2 Small", section on vLLM's optimisations) packs the query
// heads of a GQA group into one tile so that each K/V page is read once per group;
// page 2 (technical optimisations, FA4 kernel) splits the KV range, with a "sheared"
// bias access, and merges the splits.
//
// Design on gfx950:
//  * one work-group of 1, 2, 4 or 8 waves per piece of a (sequence, KV head) unit; the
//    G*n packed query rows (G = Hq/Hkv) go to 16-row MFMA tiles, one per wave (6 rows pad
//    to 16 here, not to 64 as in the pages' Blackwell tile); or waves holding RT row
//    tiles each, which read each K and V fragment from LDS once for all of them (the 48
//    rows of an 8-row verify: one wave of 3 tiles, no padding, no barrier; the 72 rows of
//    a 9-token step on 8-head groups: 4 waves of two 9-row tiles);
//  * K and V tiles of 32 keys are read with non-temporal 16-byte loads in row order (a
//    16-lane pass reads 256 contiguous bytes), two tiles in flight, and stored to LDS
//    with XOR-swizzled 16-byte chunks; page ids are staged in LDS per chunk of pages;
//  * S^T = K * Q^T on v_mfma_f32_16x16x32_bf16 with K (read back from LDS) as the A
//    operand; the S^T accumulator layout (lane = query row, 4 keys per lane) is exactly
//    the B operand layout that O^T = V^T * P^T needs, so P never moves between lanes;
//  * V is read back transposed with ds_read_b64_tr_b16, the gfx950 LDS transpose read;
//  * the bias is sheared: per tile, each head of the group needs one contiguous slice of
//    32 + n - 1 distances, which row r reads shifted by n - 1 - r; multi-wave groups load
//    the slices once (coalesced) into LDS, a single wave reads its row's entries four
//    adjacent distances per 16-byte load;
//  * online softmax in fp32, one row per lane, row max across the 4 lanes of a row, the
//    reference point moved only when a tile's maximum passes it by 8 ln 2;
//  * FP8 (OCP E4M3) K/V are decoded exactly to bf16 with v_cvt_scalef32_pk_bf16_fp8; the
//    K scale multiplies the logit column, the V scale multiplies P before its bf16
//    rounding. A tile's 64 scales arrive with one 4-byte load per lane and are staged in
//    LDS beside the tile (per-lane 16-byte scale loads cost 32 registers and 6 % of the
//    1M-key decode).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"
#include "device_common.h"

namespace rattn {

// ---------------------------------------------------------------------------------
// Split kernel: WR waves per work-group, each owning one 16-row MFMA tile of the G*n
// packed query rows of a (sequence, KV head) unit (rows per wave: ceil(G*n / WR)).
// The waves load equal shares of every 32-key K/V tile into registers, store them to
// a double-buffered LDS tile and meet at one barrier per tile; each wave then attends
// its rows over the whole tile. Each K/V byte is read from HBM once per unit.
// ---------------------------------------------------------------------------------
// Multi-wave work-groups ask for two waves per SIMD (at most 256 VGPRs each): on the
// 8-row verify workload that beat one wave per SIMD by 1.4x despite a few spilled
// registers, since every tile's barrier waits on the slowest of the group's waves.
//
// WS > 1 (single-wave pieces, bf16, a unit split into exactly WS pieces): a work-group
// holds WS waves, each attending a piece of its own exactly as a single-wave work-group
// would; the waves then merge their pieces through LDS into the unit's output, so that
// no combine launch follows (see the epilogue).
//
// RT > 1: each wave holds RT MFMA tiles of its share of the unit's packed rows (rows
// spread evenly over them). Each K fragment and V^T fragment it reads from LDS feeds RT
// matrix instructions; the queries (each wave its own block) and the tile's sheared bias
// slice are staged in LDS. A one-wave piece runs alone on its SIMD with the full register
// file and one tile in flight (the O accumulators, 32 registers per row tile, leave the
// arithmetic registers to that tile); four waves of two tiles run two waves per SIMD, two
// groups per CU, with two tiles in flight (each wave holds a quarter of a tile's loads),
// as do groups of four or eight waves of one row tile and two-wave groups of even shares
// over a bf16 cache.
// Waves per SIMD: one for a single bf16 wave (its two tiles in flight take 128 registers)
// and for a wave of row tiles (the accumulators of 2 or 3 tiles), and for 2-wave groups of
// even shares over a bf16 cache (at two per SIMD they spilled 104 bytes per lane; the
// 3-row step over 2K-8K keys at batch 16 ran 87 us at two, 73 at one); else two.
template <int WR, bool FP8, bool EVEN, int RT>
constexpr int split_kv_occupancy() {
  return (WR == 1 && (!FP8 || RT > 1)) || (WR == 2 && EVEN && !FP8 && RT == 1) ? 1 : 2;
}
#define OCCUPANCY (split_kv_occupancy<WR, FP8, EVEN, RT>())

template <int WR, bool FP8, bool EVEN, int WS, int RT>
__global__ __launch_bounds__(64 * WR * WS)
__attribute__((amdgpu_waves_per_eu(OCCUPANCY))) void split_kv_kernel(
    KernelArgs a) {
  static_assert(WS == 1 || (WR == 1 && !FP8 && !EVEN), "merging work-groups: bf16 pieces");
  static_assert(RT == 1 || WS == 1, "row tiles of a wave: not in a merging group");
  constexpr int TILE_BUFS = WR > 1 ? 2 : 1;   // LDS tile buffers (see process_tile)
  // per wave of a merging work-group (WS > 1): its own tile buffer and page ids
  __shared__ __attribute__((aligned(16))) unsigned char klds[WS * TILE_BUFS][kTileKeys * 256];
  __shared__ __attribute__((aligned(16))) unsigned char vlds[WS * TILE_BUFS][kTileKeys * 256];
  __shared__ int pages_lds[WS][kChunkPages + 1];
  // E4M3: a tile's 32 K and 32 V scales, staged beside the tile
  __shared__ __attribute__((aligned(16))) float scale_lds[FP8 ? TILE_BUFS : 1][FP8 ? 64 : 1];
  // Several waves load the bias slice of a tile together and share it through LDS, and
  // so does a wave of several row tiles; a wave of one row tile reads its row's entries
  // one tile ahead in registers, which keeps the read off each tile's critical path.
  // Both the buffer count and every index into the buffers derive from STAGE_BIAS and
  // WR (two buffers exactly when several waves share one).
  constexpr bool STAGE_BIAS = WR > 1 || RT > 1;
  constexpr int BIAS_BUFS = WR > 1 ? 2 : 1;
  constexpr int BPT = RT == 1 ? kBiasPerThread
                      : (WR == 1 ? kBiasPerThreadRows : kBiasPerThreadPair);   // slice loads per lane
  __shared__ float bias_lds[BIAS_BUFS][STAGE_BIAS ? 64 * WR * BPT : 1];
  // RT > 1: the queries of the wave's RT * 16 rows, row i's 16-byte chunk c at
  // klds_off(i, c) (the B operand reads of one instruction hit distinct banks)
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[RT > 1 ? WR : 1][RT > 1 ? RT * 16 * 256 : 16];

  const int lane = threadIdx.x & 63;
  const int wave = WR == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // WS > 1: the wave's piece within the work-group (its LDS buffers)
  const int wsi = WS == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lr = lane & 15;        // key (A operand) / query row (B operand) within a tile
  const int lq = lane >> 4;        // k-group of the MFMA operands
  const int n = a.n;
  const int G = a.group;
  const int R = G * n;
  const int S = a.page_size;
  const int W = a.window;
  const int64_t Hkv = a.num_kv_heads;
  const int rpw = (R + WR - 1) / WR;          // rows per wave
  const int rpt = RT == 1 ? rpw : (rpw + RT - 1) / RT;   // rows per row tile (<= 16)

  const int64_t wg = (int64_t)blockIdx.x * WS + wsi;   // the piece
  const int k_split = a.splits_per_unit;     // used when !EVEN
  int T = 0;
  int64_t P = 0, t_begin = 0, t_end = 0;
  if (EVEN) {                                // even shares of the whole tile space
    T = __builtin_amdgcn_readfirstlane(total_tiles(a, lane));   // the same in every lane
    P = min((int64_t)gridDim.x, (int64_t)T);
    if (wg >= P) return;                     // uniform over the work-group
    t_begin = wg * T / P;
    t_end = (wg + 1) * T / P;
  }

  // ---- this lane's query row in each of the wave's row tiles (row rho[t] of the unit's
  // packed rows): with one tile per wave, the wave's share of rpw rows; with RT tiles,
  // rows 16 t + lr ----
  int rho[RT], r_of_row[RT], hl_of_row[RT];
  bool row_ok[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    rho[t] = wave * rpw + t * rpt + lr;
    row_ok[t] = lr < rpt && t * rpt + lr < rpw && rho[t] < R;
    r_of_row[t] = row_ok[t] ? rho[t] / G : 0;
    hl_of_row[t] = row_ok[t] ? rho[t] - r_of_row[t] * G : 0;
  }

  // ---- per-tile registers: this wave's share of the tile's 16-byte loads ----
  constexpr int SLOTS = FP8 ? 8 : 16;        // 16-byte loads per lane for one whole tile
  constexpr int NSLOT = SLOTS / WR;
  struct Tile {
    u32x4_t x[NSLOT];
    float sc;    // E4M3: lane l's scale, of key l (K) or key l - 32 (V) of the tile
    // staged slices: this thread's elements of the tile's bias slice; one wave of one
    // row tile: the bias of its row for keys 4 lq + i of each subtile, gathered directly
    float bs[STAGE_BIAS ? BPT : 8];
  };
  constexpr int ROW_BYTES = FP8 ? kHeadDim : 2 * kHeadDim;
  // lane offset within a 16-key subtile block: each 16-lane pass of a load reads 256
  // contiguous bytes (one bf16 row, two E4M3 rows); a pass spread over 16 rows caps the
  // read rate near 5.2 TB/s on MI355X, against 6.4 TB/s for contiguous passes
  const unsigned kv_off = FP8 ? (lane >> 3) * 128 + 16 * (lane & 7) : lq * 256 + 16 * lr;
  const unsigned char* kc = (const unsigned char*)a.k_cache;
  const unsigned char* vc = (const unsigned char*)a.v_cache;

  // ---- merging work-groups (WS > 1): the WS pieces are the whole unit ----
  // Each wave stages its piece's normalised partial (O / l and lse per row) in its own
  // LDS tile buffer; the group merges the WS pieces by the log-sum-exp rule and writes
  // the unit's output rows. Staging layout: row rho at float offset 128 rho, its 4-float
  // chunk c at slot c ^ (rho & 15) (so that the 16 rows one store instruction writes
  // fall into distinct banks); the lse of row rho in the wave's V buffer.
  auto merge_group = [&](int b, int g, float l, float m_run, const f32x4_t (&o)[8]) {
    if constexpr (WS > 1) {
      float* st = reinterpret_cast<float*>(klds[wsi]);
      float* st_lse = reinterpret_cast<float*>(vlds[wsi]);
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int c = 4 * dt + lq;                       // dims 4 c .. 4 c + 3
        *reinterpret_cast<f32x4_t*>(st + 128 * lr + 4 * (c ^ lr)) = o[dt] * inv;
      }
      if (lq == 0) st_lse[lr] = l > 0.f ? m_run + __logf(l) : kNegInf;
      __syncthreads();

      const SeqRows sr = seq_rows(a, b, false);
      for (int idx = (int)threadIdx.x; idx < R * 32; idx += 64 * WS) {
        const int rr = idx >> 5, c = idx & 31;           // packed row, 4-dim chunk
        const int r = rr / G;
        if (r >= sr.n) continue;                         // a row the sequence lacks
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < WS; ++w)
          M = fmaxf(M, reinterpret_cast<const float*>(vlds[w])[rr]);
        float lsum = 0.f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < WS; ++w) {
          const float lw = reinterpret_cast<const float*>(vlds[w])[rr];
          const float wt = lw == kNegInf ? 0.f : __expf(lw - M);   // an empty piece: 0
          lsum += wt;
          acc += wt * *reinterpret_cast<const f32x4_t*>(
                          reinterpret_cast<const float*>(klds[w]) + 128 * rr + 4 * (c ^ (rr & 15)));
        }
        const float inv_s = lsum > 0.f ? 1.f / lsum : 0.f;
        const f32x4_t og = acc * inv_s;
        const int64_t orow = (int64_t)(sr.base + r) * a.num_q_heads + g * G + (rr - r * G);
        const u32x2_t wv = {pack_bf16x2(og[0], og[1]), pack_bf16x2(og[2], og[3])};
        *reinterpret_cast<u32x2_t*>(a.out + orow * kHeadDim + 4 * c) = wv;
        if (c == 0 && a.lse != nullptr) a.lse[orow] = lsum > 0.f ? M + __logf(lsum) : kNegInf;
      }
    }
  };

  for (bool more = true; more;) {
    // ---- the next piece: tiles [tile0, tile1) of unit (b, g) ----
    int b, g, tile0, tile1;
    SeqGeom sg;
    bool whole;
    int64_t prow0;                           // partial row of packed row 0 of the unit
    if (!EVEN) {
      const int64_t u = wg / k_split;
      const int sidx = (int)(wg - u * k_split);
      b = (int)(u / Hkv);
      g = (int)(u - (int64_t)b * Hkv);
      sg = seq_geom(a, b, true);
      tile0 = (int)((int64_t)sidx * sg.tiles / k_split);
      tile1 = (int)((int64_t)(sidx + 1) * sg.tiles / k_split);
      whole = k_split == 1;
      prow0 = wg * R;
      more = false;
      if (WS == 1 && tile1 == tile0) {
        // fewer tiles than splits: an empty piece marks its rows, which the combine
        // skips (a sequence without rows has no tiles and nothing to mark); a wave of a
        // merging work-group attends no tile and merges an empty piece (l = 0)
#pragma unroll
        for (int t = 0; t < RT; ++t)
          if (row_ok[t] && r_of_row[t] < sg.nb) a.part_lse[prow0 + rho[t]] = kNegInf;
        return;
      }
    } else {
      int before;
      locate_tile(a, lane, (int)t_begin, b, before);
      b = __builtin_amdgcn_readfirstlane(b);           // the same in every lane
      before = __builtin_amdgcn_readfirstlane(before);
      sg = seq_geom(a, b, false);
      g = (t_begin - before) / sg.tiles;
      const int64_t ustart = before + (int64_t)g * sg.tiles;
      const int64_t uend = ustart + sg.tiles;
      const int64_t piece_end = min(t_end, uend);
      tile0 = (int)(t_begin - ustart);
      tile1 = (int)(piece_end - ustart);
      whole = t_begin == ustart && piece_end == uend;
      const int64_t u = (int64_t)b * Hkv + g;
      prow0 = (wg + u) * R;
      if (t_begin == ustart && lane == 0 && wave == 0) {
        // the unit's first work-group records where its pieces are, for the combine
        // (one piece: the unit is whole and its output final)
        const int64_t w_last = (uend * P - 1) / T;
        a.unit_info[2 * u] = (int)wg;
        a.unit_info[2 * u + 1] = (int)(w_last - wg + 1);
      }
      t_begin = piece_end;
      more = t_begin < t_end;
    }
    const int L = sg.L;
    const int k_lo = sg.k_lo;
    const int nb = sg.nb;                    // this sequence's rows (<= n)
    bool row_live[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) row_live[t] = row_ok[t] && r_of_row[t] < nb;
    const int row_base = seq_rows(a, b, false).base;
    const int j_begin = sg.base + tile0 * kTileKeys;
    const int j_end = min(sg.base + tile1 * kTileKeys, L);

    // tiles at or after `fast_lo` and at or before `fast_hi` need no mask: every key is
    // visible to every row at a distance in [0, W-1]
    const int fast_lo = W > 0 ? max(0, L - W) : 0;
    const int fast_hi = L - nb - (kTileKeys - 1);
    // Bias slice (the sheared access): for a tile starting at key j0, head h of the group
    // needs distances L-1-j0-pos for pos in [0, 32+nb-1): row r reads key j at position
    // pos = (j - j0) + (nb-1-r), so the nb rows of a head share one slice, shifted by
    // their offset (the slice is sized for n >= nb rows). The group loads each head's slice once per tile, with distances
    // clamped to [0, Dmax] (a masked key reads an in-range entry that the mask
    // discards), and every lane then reads its row's entries from LDS.
    const int slice_len = kTileKeys + n - 1;
    const int slice_elems = G * slice_len;     // <= 64 WR BPT (validated)
    const int nbias = (slice_elems + 64 * WR - 1) / (64 * WR);   // slice loads per thread
    const int sub_lo = k_lo & ~15;           // first 16-key subtile holding a visible key
    const int sub_hi = (L - 1) & ~15;        // last subtile holding a key of the sequence

    int row_p[RT], bias_pos[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      row_p[t] = L - nb + r_of_row[t];
      // this lane's position in its head's slice for key 4 lq of subtile 0
      bias_pos[t] = hl_of_row[t] * slice_len + 4 * lq + max(nb - 1 - r_of_row[t], 0);
    }
    const int row_h = g * G + hl_of_row[0];
    bf16x8_t qreg[RT == 1 ? 4 : 1];
    if constexpr (RT == 1) {
      const uint16_t* qrow =
          a.q + ((int64_t)(row_base + r_of_row[0]) * a.num_q_heads + row_h) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // the K operand of MFMA s gives lane (lr, lq) the dims 32 s + 8 lq .. + 7
        const u32x4_t v = row_live[0] ? ld16(qrow + 32 * s + 8 * lq) : u32x4_t{0, 0, 0, 0};
        qreg[s] = __builtin_bit_cast(bf16x8_t, v);
      }
    } else {
      // the wave's queries into its LDS block: 16 lanes read one 256-byte row, four rows
      // per pass. Every load is issued before the first store (a tile row without a
      // query row reads the unit's first row and stores zeros), so that they share one
      // memory round trip. Each wave reads only its own block.
      u32x4_t qv[4 * RT];
      bool qlive[4 * RT];
#pragma unroll
      for (int k = 0; k < 4 * RT; ++k) {
        const int ti = 4 * k + lq;                   // tile row: tile ti / 16, row ti % 16
        const int tt = ti >> 4, tl = ti & 15;
        const int i = wave * rpw + tt * rpt + tl;    // packed row
        const int r = i / G;
        qlive[k] = tl < rpt && tt * rpt + tl < rpw && i < R && r < nb;
        const int rr = qlive[k] ? r : 0, hh = qlive[k] ? i - r * G : 0;
        qv[k] = ld16(a.q + ((int64_t)(row_base + rr) * a.num_q_heads + g * G + hh) * kHeadDim +
                     8 * lr);
      }
#pragma unroll
      for (int k = 0; k < 4 * RT; ++k) {
        const unsigned keep = qlive[k] ? ~0u : 0u;
        *reinterpret_cast<u32x4_t*>(q_lds[RT > 1 ? wave : 0] + klds_off(4 * k + lq, lr)) =
            qv[k] & u32x4_t{keep, keep, keep, keep};
      }
    }
    // the row's table offset (for the direct gather of a one-tile wave)
    const int bias_row = row_h * (a.dmax + 1);
    // this thread's slice elements: element e = tid + 64 WR q of the group's slices is
    // position e % slice_len of head e / slice_len; bs_row is that head's table offset
    // (-1: no element), bs_pos the position
    int bs_row[BPT], bs_pos[BPT];
    {
      const int tid = wave * 64 + lane;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        const int e = tid + 64 * WR * q;
        const int hl = e / slice_len;
        bs_pos[q] = e - hl * slice_len;
        bs_row[q] = e < slice_elems ? (g * G + hl) * (a.dmax + 1) : -1;
      }
    }

    // ---- page ids ----
    // The ids of the pages a chunk of the piece touches are staged in LDS before its
    // tile loop, so that the loop looks them up with an LDS read: a page-table load in
    // the loop would make every tile wait for all of its predecessors' K/V loads.
    const int32_t* pt_row = a.page_table + (int64_t)b * a.max_pages;
    int chunk_p0 = 0;
    // The ids are loaded in batches of up to four per thread, each batch issued before
    // its first id is checked (an index past the chunk re-reads its last id), so that a
    // batch costs one memory round trip.
    constexpr int PAGE_BATCH = 4;
    auto stage_pages = [&](int c0, int c1) {
      if (WR > 1) __syncthreads();           // the previous chunk's ids and tiles are done
      chunk_p0 = c0 >> a.page_shift;
      const int np = ((c1 - 1) >> a.page_shift) - chunk_p0 + 1;   // <= kChunkPages + 1
      const int tid = WS > 1 ? lane : (int)threadIdx.x;
      for (int i0 = 0; i0 < np; i0 += 64 * WR * PAGE_BATCH) {   // uniform
        int ids[PAGE_BATCH];
#pragma unroll
        for (int k = 0; k < PAGE_BATCH; ++k)
          ids[k] = pt_row[chunk_p0 + min(i0 + tid + 64 * WR * k, np - 1)];
#pragma unroll
        for (int k = 0; k < PAGE_BATCH; ++k) {
          const int i = i0 + tid + 64 * WR * k;
          int ph = ids[k];
          if (ph < 0 || ph >= a.num_pages) {
            atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
            ph = min(max(ph, 0), a.num_pages - 1);
          }
          if (i < np) pages_lds[wsi][i] = ph;
        }
      }
      if (WR > 1) __syncthreads();
    };
    auto phys_at = [&](int jt) -> int {     // physical page of key jt of the current chunk
      const int idx = min(max((jt >> a.page_shift) - chunk_p0, 0), kChunkPages);
      return __builtin_amdgcn_readfirstlane(pages_lds[wsi][idx]);
    };

    // Every load of a tile is issued unconditionally, so that the compiler can count the
    // loads in flight and wait for exactly one tile at a time. A subtile with no key in
    // [k_lo, L) (at the two ends of the visible range) reads the nearest subtile that
    // has one instead; the masks of process_tile discard its keys.
    auto load_tile = [&](Tile& X, int j0) {
      if constexpr (STAGE_BIAS) {
        // the bias slice elements of this thread (a thread without one re-reads entry 0),
        // through the caches: the sequences of a batch read the same distances (the
        // 8-row verify workload reads 1.04x its algorithmic bytes this way, 1.08x with
        // non-temporal loads)
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
          if (q > 0 && q >= nbias) break;   // uniform
          const int d = min(max(L - 1 - j0 - bs_pos[q], 0), a.dmax);
          X.bs[q] = a.bias[bs_row[q] >= 0 ? (unsigned)(bs_row[q] + d) : 0u];
        }
      }
      int64_t tok0[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int js = min(max(j0 + 16 * kt, sub_lo), sub_hi);
        tok0[kt] = ((int64_t)phys_at(js) * Hkv + g) * S + (js & (S - 1));
      }
#pragma unroll
      for (int m = 0; m < NSLOT; ++m) {
        // slot = (K|V, subtile, 1 KiB block of the subtile)
        const int slot = wave + WR * m;
        const int kv = FP8 ? slot >> 2 : slot >> 3;
        const int kt = FP8 ? (slot >> 1) & 1 : (slot >> 2) & 1;
        const int u = FP8 ? slot & 1 : slot & 3;
        const unsigned char* base = (kv ? vc : kc) + tok0[kt] * ROW_BYTES;
        X.x[m] = ld16_stream(base + kv_off + 1024 * u);
      }
      if (FP8) {
        // one 4-byte load per lane: the tile's 32 K scales, then its 32 V scales
        const int64_t tok = ((lane & 16) ? tok0[1] : tok0[0]) + (lane & 15);
        X.sc = __builtin_nontemporal_load((lane & 32 ? a.v_scale : a.k_scale) + tok);
      }
      if constexpr (!STAGE_BIAS) {
        // row r of head h reads B[h][p_r - j] for its keys j = j0 + 16 kt + 4 lq + i: the
        // four distances d0 - i (d0 = p_r - j0 - 16 kt - 4 lq) are adjacent table entries,
        // read with one 16-byte load when all four lie in [0, Dmax] (four times fewer
        // vector-memory instructions), else one by one with the distances clamped
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int d0 = row_p[0] - (j0 + 16 * kt + 4 * lq);
          if (d0 >= 3 && d0 <= a.dmax) {
            const f32x4_t v = ldf4u_stream(a.bias + (unsigned)(bias_row + d0 - 3));
#pragma unroll
            for (int i = 0; i < 4; ++i) X.bs[4 * kt + i] = v[3 - i];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int d = min(max(d0 - i, 0), a.dmax);
              X.bs[4 * kt + i] = ldf_stream(a.bias + (unsigned)(bias_row + d));
            }
          }
        }
      }
    };

    // ---- running state of this lane's row in each row tile ----
    f32x4_t o[RT][8];
    float m_run[RT], l_run[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      m_run[t] = kNegInf;
      l_run[t] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4_t{0, 0, 0, 0};
    }

    // A tile is attended in two steps: its registers are stored to LDS (stage_tile), then
    // the wave computes from LDS (attend_tile); between the two the registers are free
    // for the next tile's loads.
    auto stage_tile = [&](const Tile& X, int j0, int buf) {
      const bool fast = (j0 >= fast_lo) && (j0 <= fast_hi);   // uniform
      // a single wave reuses one LDS buffer (its LDS accesses execute in order); several
      // waves alternate two, so that one barrier per tile separates writes from reads
      unsigned char* kl = klds[wsi * TILE_BUFS + (TILE_BUFS == 2 ? buf : 0)];
      unsigned char* vl = vlds[wsi * TILE_BUFS + (TILE_BUFS == 2 ? buf : 0)];
      float* bl = bias_lds[BIAS_BUFS == 2 ? buf : 0];
      if constexpr (STAGE_BIAS) {
        const int tid = wave * 64 + lane;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
          if (q > 0 && q >= nbias) break;   // uniform
          bl[tid + 64 * WR * q] = X.bs[q];   // in the buffer; past the slice: unread
        }
      }
      // this wave's share -> LDS as bf16 (swizzled). V of keys outside [k_lo, L) becomes
      // zero, so that P = 0 times a stale or NaN value cannot reach the accumulator.
#pragma unroll
      for (int m = 0; m < NSLOT; ++m) {
        const int slot = wave + WR * m;
        const int kv = FP8 ? slot >> 2 : slot >> 3;
        const int kt = FP8 ? (slot >> 1) & 1 : (slot >> 2) & 1;
        const int u = FP8 ? slot & 1 : slot & 3;
        if (!FP8) {
          const int kk = 16 * kt + 4 * u + lq;
          u32x4_t v = X.x[m];
          if (kv == 0) {
            *reinterpret_cast<u32x4_t*>(kl + klds_off(kk, lr)) = v;
          } else {
            const int j = j0 + kk;
            if (!fast) {                                // uniform; inside, a mask
              const unsigned keep = (j < k_lo || j >= L) ? 0u : ~0u;
              v &= u32x4_t{keep, keep, keep, keep};
            }
            *reinterpret_cast<u32x4_t*>(vl + vlds_off(kk, lr)) = v;
          }
        } else {
          const int kk = 16 * kt + 8 * u + (lane >> 3);
          const int c8 = lane & 7;
          u32x4_t raw = X.x[m];
          if (kv == 1) {
            const int j = j0 + kk;
            if (!fast) {
              const unsigned keep = (j < k_lo || j >= L) ? 0u : ~0u;
              raw &= u32x4_t{keep, keep, keep, keep};
            }
          }
          const u32x2_t c0 = e4m3x4_to_bf16x4(raw.x), c1 = e4m3x4_to_bf16x4(raw.y);
          const u32x2_t c2 = e4m3x4_to_bf16x4(raw.z), c3 = e4m3x4_to_bf16x4(raw.w);
          const u32x4_t lo = {c0.x, c0.y, c1.x, c1.y}, hi = {c2.x, c2.y, c3.x, c3.y};
          if (kv == 0) {
            *reinterpret_cast<u32x4_t*>(kl + klds_off(kk, 2 * c8)) = lo;
            *reinterpret_cast<u32x4_t*>(kl + klds_off(kk, 2 * c8 + 1)) = hi;
          } else {
            *reinterpret_cast<u32x4_t*>(vl + vlds_off(kk, 2 * c8)) = lo;
            *reinterpret_cast<u32x4_t*>(vl + vlds_off(kk, 2 * c8 + 1)) = hi;
          }
        }
      }
      float* sl = scale_lds[FP8 && TILE_BUFS == 2 ? buf : 0];
      if (FP8 && wave == 0) sl[lane] = X.sc;
      if (WR > 1) __syncthreads();            // the whole tile is in LDS buffer `buf`
    };

    auto attend_tile = [&](const Tile& X, int j0, int buf) {
      const bool fast = (j0 >= fast_lo) && (j0 <= fast_hi);   // uniform
      const unsigned char* kl = klds[wsi * TILE_BUFS + (TILE_BUFS == 2 ? buf : 0)];
      const unsigned char* vl = vlds[wsi * TILE_BUFS + (TILE_BUFS == 2 ? buf : 0)];
      const float* bl = bias_lds[BIAS_BUFS == 2 ? buf : 0];
      const float* sl = scale_lds[FP8 && TILE_BUFS == 2 ? buf : 0];
      (void)bl;
      (void)sl;

      // S^T = K Q^T : lane (lr, lq) of MFMA s reads key 16 kt + lr, dims 32 s + 8 lq ..;
      // the result gives lane (lr, lq) row lr and keys 4 lq + i of each 16-key subtile.
      // Each K fragment feeds the MFMAs of all the wave's row tiles.
      f32x4_t sacc[RT][2];
#pragma unroll
      for (int t = 0; t < RT; ++t) sacc[t][0] = sacc[t][1] = f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t kop[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          kop[kt] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(kl + klds_off(16 * kt + lr, 4 * s + lq)));
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          bf16x8_t qop;
          if constexpr (RT == 1) qop = qreg[s];
          else
            qop = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t*>(q_lds[RT > 1 ? wave : 0] +
                                                            klds_off(16 * t + lr, 4 * s + lq)));
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            sacc[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt], qop, sacc[t][kt], 0, 0, 0);
        }
      }

      // Several row tiles: the scheduler may not move the work of one phase (logits,
      // softmax, PV) into another, so that each phase's temporaries die before the next
      // one's are made (with the full register file of a lone wave it otherwise hoists
      // the V^T reads and the next tile's work until the accumulators spill).
      if constexpr (RT > 1) __builtin_amdgcn_sched_barrier(0);

      // E4M3: the scales of this lane's keys 4 lq + i of each subtile
      f32x4_t ks[2], vs[2];
      if constexpr (FP8) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          ks[kt] = *reinterpret_cast<const f32x4_t*>(sl + 16 * kt + 4 * lq);
          vs[kt] = *reinterpret_cast<const f32x4_t*>(sl + 32 + 16 * kt + 4 * lq);
        }
      }

      // per row tile: bias, logits, mask, online softmax; P packed as the B operand of
      // O^T += V^T P^T
      bf16x8_t pop[RT], pop_lo[FP8 ? RT : 1];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        // the bias of this lane's row for its keys 4 lq + i of each subtile
        float bv[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (STAGE_BIAS) bv[kt][i] = bl[bias_pos[t] + 16 * kt + i];
            else bv[kt][i] = X.bs[4 * kt + i];
          }
        // the logits and this lane's maximum; the masks only on tiles at the edges of
        // the visible range (one uniform branch around each form of the loop)
        float sv[2][4];
        float mt = kNegInf;
        if (fast) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float scl = FP8 ? a.softmax_scale * ks[kt][i] : a.softmax_scale;
              sv[kt][i] = __builtin_fmaf(sacc[t][kt][i], scl, bv[kt][i]);
              mt = fmaxf(mt, sv[kt][i]);
            }
        } else {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float scl = FP8 ? a.softmax_scale * ks[kt][i] : a.softmax_scale;
              const float sc = __builtin_fmaf(sacc[t][kt][i], scl, bv[kt][i]);
              const int dist = row_p[t] - (j0 + 16 * kt + 4 * lq + i);
              const bool vis = row_live[t] && dist >= 0 && (W == 0 || dist < W);
              sv[kt][i] = vis ? sc : kNegInf;
              mt = fmaxf(mt, sv[kt][i]);
            }
        }
        // The reference point m of a row moves only when the tile's maximum exceeds it
        // by more than kRescaleSlack, so that the accumulators are rescaled on few
        // tiles; p = exp(s - m) then stays below exp(kRescaleSlack). O and l share m, so
        // the quotient O / l and lse = m + ln l are unchanged by the choice of m. The
        // test runs on each lane's own maximum: a row's maximum passes m + kRescaleSlack
        // exactly when the maximum of one of its 4 lanes does, so the row maximum is
        // taken (across the lanes) only in the rare branch.
        if (__ballot(mt > m_run[t] + kRescaleSlack) != 0) {   // wave-uniform; false at -inf
          mt = wave_max_rows(mt);
          const bool grow = mt > m_run[t] + kRescaleSlack;
          const float m_new = grow ? mt : m_run[t];
          const float alpha = grow ? __builtin_amdgcn_exp2f((m_run[t] - m_new) * kLog2e) : 1.f;
          l_run[t] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[t][dt] *= alpha;
          m_run[t] = m_new;
        }
        const float mb = -(m_run[t] == kNegInf ? 0.f : m_run[t]) * kLog2e;
        float psum = 0.f;
        float pv[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kt][i], kLog2e, mb));
            psum += p;
            pv[kt][i] = FP8 ? (p > 0.f ? p * vs[kt][i] : 0.f) : p;
          }
        }
        l_run[t] += psum;
        const u32x4_t pk = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                            pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
        pop[t] = __builtin_bit_cast(bf16x8_t, pk);
        if constexpr (FP8) {
          // P times the V scales is not a bf16 value: its rounding remainder goes to the
          // matrix units too (a second PV product), so that one visible key gives its
          // value to within the output's own bf16 rounding
          const u32x4_t pr = {pack_bf16x2_rem(pv[0][0], pv[0][1], pk.x),
                              pack_bf16x2_rem(pv[0][2], pv[0][3], pk.y),
                              pack_bf16x2_rem(pv[1][0], pv[1][1], pk.z),
                              pack_bf16x2_rem(pv[1][2], pv[1][3], pk.w)};
          pop_lo[t] = __builtin_bit_cast(bf16x8_t, pr);
        }
      }

      if constexpr (RT > 1) __builtin_amdgcn_sched_barrier(0);

      // O^T += V^T P^T : V^T operand by transpose reads of the LDS tile. Lane (lr, lq)
      // supplies the address of 4 dims of key 16 e + 4 lq + lr/4; the read returns to
      // lane lr the dim 16 dt + lr of keys 16 e + 4 lq + 0..3. Each V^T fragment feeds
      // the MFMAs of all the wave's row tiles.
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int cc = 2 * dt + ((lr & 3) >> 1);
        const int k0 = 4 * lq + (lr >> 2);
        const int off0 = vlds_off(k0, cc) + 8 * (lr & 1);
        const int off1 = vlds_off(16 + k0, cc) + 8 * (lr & 1);
        const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3)))*)(vl + off0));
        const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3)))*)(vl + off1));
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, v0), w1 = __builtin_bit_cast(u32x2_t, v1);
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, u32x4_t{w0.x, w0.y, w1.x, w1.y});
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t], o[t][dt], 0, 0, 0);
          if constexpr (FP8)
            o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo[t], o[t][dt], 0, 0, 0);
        }
      }
    };

    auto process_tile = [&](const Tile& X, int j0, int buf) {
      stage_tile(X, j0, buf);
      attend_tile(X, j0, buf);
    };

    // ---- tile loop, chunks of at most kChunkPages pages. Groups of four or eight waves
    // (each wave a quarter or an eighth of a tile's loads), and two waves of even shares
    // over a bf16 cache (one per SIMD): two tiles in flight while one is attended. One
    // wave, or two waves at two per SIMD, of one row tile: two tiles in registers, the
    // next tile's loads in flight while one is attended. Several row tiles in a lone wave
    // (their accumulators take the registers): one tile in flight, whose loads are issued
    // as soon as the tile before it is in LDS, so that they are in flight while the wave
    // attends that tile ----
    const int chunk_keys = (int)min((int64_t)kChunkPages * S, (int64_t)1 << 30);
    constexpr bool TWO_AHEAD = (RT > 1 && WR > 1) || WR >= 4 || (WR == 2 && EVEN && !FP8);
    constexpr bool ONE_IN_FLIGHT = RT > 1 && !TWO_AHEAD;
    if constexpr (TWO_AHEAD) {
      // Two tiles in flight while one is attended, in registers A and B by turns. (Over
      // short pieces, as in a window layer's verify, a tile's loads then wait less; a lone
      // wave, whose share of a tile is the whole tile, keeps the other loop.) Each tile's loads are
      // issued right after the tile two places before it is in LDS. In the steady state
      // every load is issued without a condition, so that the compiler waits for exactly
      // one tile; a chunk of fewer than two tiles loads its one tile twice.
      Tile A, B;
      for (int c0 = j_begin; c0 < j_end; c0 += chunk_keys) {
        const int c1 = min(c0 + chunk_keys, j_end);
        stage_pages(c0, c1);
        const int nt = (c1 - c0 + kTileKeys - 1) / kTileKeys;
        load_tile(A, c0);
        load_tile(B, c0 + min(1, nt - 1) * kTileKeys);
        int i = 0;
        for (; i + 4 <= nt; i += 2) {
          const int j0 = c0 + i * kTileKeys;
          stage_tile(A, j0, 0);
          load_tile(A, j0 + 2 * kTileKeys);
          attend_tile(A, j0, 0);
          stage_tile(B, j0 + kTileKeys, 1);
          load_tile(B, j0 + 3 * kTileKeys);
          attend_tile(B, j0 + kTileKeys, 1);
        }
        // the last 1, 2 or 3 tiles (uniform), tile i in A and tile i + 1 in B
        const int j0 = c0 + i * kTileKeys;
        const int rest = nt - i;
        stage_tile(A, j0, 0);
        if (rest == 3) load_tile(A, j0 + 2 * kTileKeys);
        attend_tile(A, j0, 0);
        if (rest >= 2) {
          process_tile(B, j0 + kTileKeys, 1);
          if (rest == 3) process_tile(A, j0 + 2 * kTileKeys, 0);
        }
      }
    }
    if constexpr (ONE_IN_FLIGHT) {
      Tile A;
      for (int c0 = j_begin; c0 < j_end; c0 += chunk_keys) {
        const int c1 = min(c0 + chunk_keys, j_end);
        stage_pages(c0, c1);
        const int nt = (c1 - c0 + kTileKeys - 1) / kTileKeys;
        load_tile(A, c0);
        for (int i = 0; i < nt; ++i) {
          const int j0 = c0 + i * kTileKeys;
          stage_tile(A, j0, 0);              // a lone wave: one LDS tile buffer
          if (i + 1 < nt) load_tile(A, j0 + kTileKeys);
          attend_tile(A, j0, i & 1);
        }
      }
    }
    // Two tiles in registers: the loads of tile i + 1 are issued before tile i is staged.
    Tile A, B;
    for (int c0 = j_begin; RT == 1 && !TWO_AHEAD && c0 < j_end; c0 += chunk_keys) {
      const int c1 = min(c0 + chunk_keys, j_end);
      stage_pages(c0, c1);
      const int nt = (c1 - c0 + kTileKeys - 1) / kTileKeys;
      load_tile(A, c0);
      int i = 0;
      for (; i + 3 <= nt; i += 2) {
        const int j0 = c0 + i * kTileKeys;
        load_tile(B, j0 + kTileKeys);
        process_tile(A, j0, 0);
        load_tile(A, j0 + 2 * kTileKeys);
        process_tile(B, j0 + kTileKeys, 1);
      }
      if (i + 2 == nt) {              // the last one or two tiles of the chunk
        const int j0 = c0 + i * kTileKeys;
        load_tile(B, j0 + kTileKeys);
        process_tile(A, j0, 0);
        process_tile(B, j0 + kTileKeys, 1);
      } else {
        process_tile(A, c0 + i * kTileKeys, 0);
      }
    }

    // ---- epilogue: the final rows when the piece is the whole unit, else partials ----
    if constexpr (WS > 1) {
      merge_group(b, g, wave_sum_rows(l_run[0]), m_run[0], o[0]);
      return;
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const float l = wave_sum_rows(l_run[t]);
      if (!row_live[t]) continue;
      const int64_t row =
          (int64_t)(row_base + r_of_row[t]) * a.num_q_heads + g * G + hl_of_row[t];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float lse = l > 0.f ? m_run[t] + __logf(l) : kNegInf;
      if (whole) {
        uint16_t* op = a.out + row * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const f32x4_t v = o[t][dt] * inv;
          const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2_t*>(op + 16 * dt + 4 * lq) = w;
        }
        if (lq == 0 && a.lse != nullptr) a.lse[row] = lse;
      } else {
        const int64_t prow = prow0 + rho[t];
        float* pp = a.part_o + prow * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<f32x4_t*>(pp + 16 * dt + 4 * lq) = o[t][dt] * inv;
        if (lq == 0) a.part_lse[prow] = lse;
      }
    }
  }
}

}  // namespace rattn
