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
//  * the bias is sheared: per tile, each head of the group needs one contiguous slice of
//    32 + n - 1 distances, which row r reads shifted by r; the work-group loads the
//    slices once (coalesced) into LDS and each lane reads its row's entries there;
//  * online softmax in fp32, one row per lane, row max across the 4 lanes of a row;
//  * FP8 (OCP E4M3) K/V are decoded exactly to bf16 with v_cvt_scalef32_pk_bf16_fp8; the K scale
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
template <int WR, bool FP8, bool EVEN>
__global__ __launch_bounds__(64 * WR)
__attribute__((amdgpu_waves_per_eu(WR == 1 && !FP8 ? 1 : 2))) void split_kv_kernel(KernelArgs a) {
  constexpr int TILE_BUFS = WR > 1 ? 2 : 1;   // LDS tile buffers (see process_tile)
  __shared__ __attribute__((aligned(16))) unsigned char klds[TILE_BUFS][kTileKeys * 256];
  __shared__ __attribute__((aligned(16))) unsigned char vlds[TILE_BUFS][kTileKeys * 256];
  __shared__ int pages_lds[kChunkPages + 1];
  // Several waves load the bias slice of a tile together and share it through LDS; a
  // single wave gathers its row's entries one tile ahead in registers, which keeps the
  // read off each tile's critical path. Both the buffer count and every index into the
  // buffers derive from STAGE_BIAS (two buffers exactly when several waves share one).
  constexpr bool STAGE_BIAS = WR > 1;
  constexpr int BIAS_BUFS = STAGE_BIAS ? 2 : 1;
  __shared__ float bias_lds[BIAS_BUFS][STAGE_BIAS ? kMaxBiasSlice : 1];

  const int lane = threadIdx.x & 63;
  const int wave = WR == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lr = lane & 15;        // key (A operand) / query row (B operand) within a tile
  const int lq = lane >> 4;        // k-group of the MFMA operands
  const int n = a.n;
  const int G = a.group;
  const int R = G * n;
  const int S = a.page_size;
  const int W = a.window;
  const int64_t Hkv = a.num_kv_heads;
  const int rpw = (R + WR - 1) / WR;

  const int64_t wg = blockIdx.x;
  const int k_split = a.splits_per_unit;     // used when !EVEN
  int T = 0;
  int64_t P = 0, t_begin = 0, t_end = 0;
  if (EVEN) {                                // even shares of the whole tile space
    T = total_tiles(a, lane);
    P = min((int64_t)gridDim.x, (int64_t)T);
    if (wg >= P) return;                     // uniform over the work-group
    t_begin = wg * T / P;
    t_end = (wg + 1) * T / P;
  }

  // ---- this wave's query row (row rho of the unit's packed rows) ----
  const int rho = wave * rpw + lr;
  const bool row_ok = lr < rpw && rho < R;
  const int r_of_row = row_ok ? rho / G : 0;
  const int hl_of_row = row_ok ? rho - r_of_row * G : 0;

  // ---- per-tile registers: this wave's share of the tile's 16-byte loads ----
  constexpr int SLOTS = FP8 ? 8 : 16;        // 16-byte loads per lane for one whole tile
  constexpr int NSLOT = SLOTS / WR;
  struct Tile {
    u32x4_t x[NSLOT];
    f32x4_t ks[2], vs[2];
    // multi-wave groups: this thread's elements of the tile's bias slice; one wave:
    // the bias of its row for keys 4 lq + i of each subtile, gathered directly
    float bs[STAGE_BIAS ? kBiasPerThread : 8];
  };
  constexpr int ROW_BYTES = FP8 ? kHeadDim : 2 * kHeadDim;
  // lane offset within a 16-key subtile block: each 16-lane pass of a load reads 256
  // contiguous bytes (one bf16 row, two E4M3 rows); a pass spread over 16 rows caps the
  // read rate near 5.2 TB/s on MI355X, against 6.4 TB/s for contiguous passes
  const unsigned kv_off = FP8 ? (lane >> 3) * 128 + 16 * (lane & 7) : lq * 256 + 16 * lr;
  const unsigned sc_off = 16 * lq;
  const unsigned char* kc = (const unsigned char*)a.k_cache;
  const unsigned char* vc = (const unsigned char*)a.v_cache;

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
      if (tile1 == tile0) {
        // fewer tiles than splits: an empty piece marks its rows, which the combine
        // skips (a sequence without rows has no tiles and nothing to mark)
        if (row_ok && r_of_row < sg.nb) a.part_lse[prow0 + rho] = kNegInf;
        return;
      }
    } else {
      int before;
      locate_tile(a, lane, (int)t_begin, b, before);
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
    const bool row_live = row_ok && r_of_row < nb;
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
    const int slice_elems = G * slice_len;     // <= kMaxBiasSlice (validated)
    const int sub_lo = k_lo & ~15;           // first 16-key subtile holding a visible key
    const int sub_hi = (L - 1) & ~15;        // last subtile holding a key of the sequence

    const int row_h = g * G + hl_of_row;
    const int row_p = L - nb + r_of_row;
    bf16x8_t qreg[4];
    {
      const uint16_t* qrow =
          a.q + ((int64_t)(row_base + r_of_row) * a.num_q_heads + row_h) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // the K operand of MFMA s gives lane (lr, lq) the dims 32 s + 8 lq .. + 7
        const u32x4_t v = row_live ? ld16(qrow + 32 * s + 8 * lq) : u32x4_t{0, 0, 0, 0};
        qreg[s] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    // this lane's position in its head's slice for key 4 lq of subtile 0, and its row's
    // table offset (for the direct gather)
    const int bias_pos = hl_of_row * slice_len + 4 * lq + max(nb - 1 - r_of_row, 0);
    const int bias_row = row_h * (a.dmax + 1);
    // this thread's slice elements: element e = tid + 64 WR q of the group's slices is
    // position e % slice_len of head e / slice_len; bs_row is that head's table offset
    // (-1: no element), bs_pos the position
    int bs_row[kBiasPerThread], bs_pos[kBiasPerThread];
    {
      const int tid = wave * 64 + lane;
#pragma unroll
      for (int q = 0; q < kBiasPerThread; ++q) {
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
    auto stage_pages = [&](int c0, int c1) {
      if (WR > 1) __syncthreads();           // the previous chunk's ids and tiles are done
      chunk_p0 = c0 >> a.page_shift;
      const int np = ((c1 - 1) >> a.page_shift) - chunk_p0 + 1;   // <= kChunkPages + 1
      for (int i = (int)threadIdx.x; i < np; i += 64 * WR) {
        int ph = pt_row[chunk_p0 + i];
        if (ph < 0 || ph >= a.num_pages) {
          atomicOr(a.flags, RATTN_FLAG_PAGE_CLAMPED);
          ph = min(max(ph, 0), a.num_pages - 1);
        }
        pages_lds[i] = ph;
      }
      if (WR > 1) __syncthreads();
    };
    auto phys_at = [&](int jt) -> int {     // physical page of key jt of the current chunk
      const int idx = min(max((jt >> a.page_shift) - chunk_p0, 0), kChunkPages);
      return __builtin_amdgcn_readfirstlane(pages_lds[idx]);
    };

    // Every load of a tile is issued unconditionally, so that the compiler can count the
    // loads in flight and wait for exactly one tile at a time. A subtile with no key in
    // [k_lo, L) (at the two ends of the visible range) reads the nearest subtile that
    // has one instead; the masks of process_tile discard its keys.
    auto load_tile = [&](Tile& X, int j0) {
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
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          X.ks[kt] = __builtin_nontemporal_load(
              (const f32x4_t*)((const unsigned char*)(a.k_scale + tok0[kt]) + sc_off));
          X.vs[kt] = __builtin_nontemporal_load(
              (const f32x4_t*)((const unsigned char*)(a.v_scale + tok0[kt]) + sc_off));
        }
      }
      if constexpr (STAGE_BIAS) {
        // the bias slice elements of this thread (a thread without one re-reads entry 0)
#pragma unroll
        for (int q = 0; q < kBiasPerThread; ++q) {
          const int d = min(max(L - 1 - j0 - bs_pos[q], 0), a.dmax);
          X.bs[q] = ldf_stream(a.bias + (bs_row[q] >= 0 ? (unsigned)(bs_row[q] + d) : 0u));
        }
      } else {
        // row r of head h reads B[h][p_r - j] for its keys, distances clamped to [0, Dmax]
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = min(max(row_p - (j0 + 16 * kt + 4 * lq + i), 0), a.dmax);
            X.bs[4 * kt + i] = ldf_stream(a.bias + (unsigned)(bias_row + d));
          }
      }
    };

    // ---- running state of this lane's row ----
    f32x4_t o[8];
    float m_run = kNegInf, l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0, 0, 0, 0};

    auto process_tile = [&](const Tile& X, int j0, int buf) {
      const bool fast = (j0 >= fast_lo) && (j0 <= fast_hi);   // uniform
      // a single wave reuses one LDS buffer (its LDS accesses execute in order); several
      // waves alternate two, so that one barrier per tile separates writes from reads
      unsigned char* kl = klds[TILE_BUFS == 2 ? buf : 0];
      unsigned char* vl = vlds[TILE_BUFS == 2 ? buf : 0];
      float* bl = bias_lds[BIAS_BUFS == 2 ? buf : 0];
      if constexpr (STAGE_BIAS) {
        const int tid = wave * 64 + lane;
#pragma unroll
        for (int q = 0; q < kBiasPerThread; ++q)
          if (bs_row[q] >= 0) bl[tid + 64 * WR * q] = X.bs[q];
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
            if (!fast && (j < k_lo || j >= L)) v = u32x4_t{0, 0, 0, 0};
            *reinterpret_cast<u32x4_t*>(vl + vlds_off(kk, lr)) = v;
          }
        } else {
          const int kk = 16 * kt + 8 * u + (lane >> 3);
          const int c8 = lane & 7;
          u32x4_t raw = X.x[m];
          if (kv == 1) {
            const int j = j0 + kk;
            if (!fast && (j < k_lo || j >= L)) raw = u32x4_t{0, 0, 0, 0};
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
      if (WR > 1) __syncthreads();            // the whole tile is in LDS buffer `buf`

      // S^T = K Q^T : lane (lr, lq) of MFMA s reads key 16 kt + lr, dims 32 s + 8 lq ..;
      // the result gives lane (lr, lq) row lr and keys 4 lq + i of each 16-key subtile
      f32x4_t sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t kop = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(kl + klds_off(16 * kt + lr, 4 * s + lq)));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[s], acc, 0, 0, 0);
        }
        sacc[kt] = acc;
      }

      // the bias of this lane's row for its keys 4 lq + i of each subtile
      float bv[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (STAGE_BIAS) bv[kt][i] = bl[bias_pos + 16 * kt + i];
          else bv[kt][i] = X.bs[4 * kt + i];
        }

      // logits, mask, online softmax; P packed as the B operand of O^T += V^T P^T
      float sv[2][4];
      float mt = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float scl = FP8 ? a.softmax_scale * X.ks[kt][i] : a.softmax_scale;
          float sc = __builtin_fmaf(sacc[kt][i], scl, bv[kt][i]);
          if (!fast) {
            const int dist = row_p - (j0 + 16 * kt + 4 * lq + i);
            const bool vis = row_live && dist >= 0 && (W == 0 || dist < W);
            sc = vis ? sc : kNegInf;
          }
          sv[kt][i] = sc;
          mt = fmaxf(mt, sc);
        }
      }
      mt = wave_max_rows(mt);
      // The reference point m of a row moves only when the tile's maximum exceeds it by
      // more than kRescaleSlack, so that the accumulators are rescaled on few tiles;
      // p = exp(s - m) then stays below exp(kRescaleSlack). O and l share m, so the
      // quotient O / l and lse = m + ln l are unchanged by the choice of m.
      const bool grow = mt > m_run + kRescaleSlack;      // false while mt = -inf
      if (__ballot(grow) != 0) {                         // wave-uniform
        const float m_new = grow ? mt : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      const float mb = -(m_run == kNegInf ? 0.f : m_run) * kLog2e;
      float psum = 0.f;
      float pv[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kt][i], kLog2e, mb));
          psum += p;
          pv[kt][i] = FP8 ? (p > 0.f ? p * X.vs[kt][i] : 0.f) : p;
        }
      }
      l_run += psum;
      const u32x4_t pk = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                          pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};
      const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pk);

      // O^T += V^T P^T : V^T operand by transpose reads of the LDS tile. Lane (lr, lq)
      // supplies the address of 4 dims of key 16 e + 4 lq + lr/4; the read returns to
      // lane lr the dim 16 dt + lr of keys 16 e + 4 lq + 0..3.
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
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, o[dt], 0, 0, 0);
      }
    };

    // ---- tile loop: two tiles in flight, chunks of at most kChunkPages pages ----
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

    // ---- epilogue: the final row when the piece is the whole unit, else a partial ----
    const float l = wave_sum_rows(l_run);
    if (row_live) {
      const int64_t row = (int64_t)(row_base + r_of_row) * a.num_q_heads + row_h;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float lse = l > 0.f ? m_run + __logf(l) : kNegInf;
      if (whole) {
        uint16_t* op = a.out + row * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const f32x4_t v = o[dt] * inv;
          const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2_t*>(op + 16 * dt + 4 * lq) = w;
        }
        if (lq == 0 && a.lse != nullptr) a.lse[row] = lse;
      } else {
        const int64_t prow = prow0 + rho;
        float* pp = a.part_o + prow * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<f32x4_t*>(pp + 16 * dt + 4 * lq) = o[dt] * inv;
        if (lq == 0) a.part_lse[prow] = lse;
      }
    }
  }
}

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
//   * few pieces per unit: 32 lanes (1 stripe) or 64 (2 stripes) cover a whole row;
//   * tens of pieces: 8 stripes x 8 lanes per 32-dim slice of a row, one wave each;
//   * hundreds of pieces: 128 stripes per 32-dim slice, 16 waves (8 pieces in flight
//     per thread, which fits the 128 registers of a 1024-thread work-group).
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

// ---------------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------------
// variant index: waves (1, 2, 4), KV format, partition
#define RATTN_VARIANTS(X)                                                               \
  X(1, false, false) X(1, true, false) X(2, false, false) X(2, true, false)              \
  X(4, false, false) X(4, true, false) X(1, false, true) X(1, true, true)                \
  X(2, false, true) X(2, true, true) X(4, false, true) X(4, true, true)

static int variant_key(int waves, bool fp8, bool even) {
  return waves * 4 + (fp8 ? 2 : 0) + (even ? 1 : 0);
}

int launch_split_kv(const KernelArgs& a, int waves, bool fp8, void* stream) {
  const dim3 grid((unsigned)a.split_groups);
  const hipStream_t st = (hipStream_t)stream;
  const int key = variant_key(waves, fp8, a.splits_per_unit == 0);
#define RATTN_LAUNCH(WRV, F8, EV)                                                    \
  if (key == variant_key(WRV, F8, EV)) {                                             \
    hipLaunchKernelGGL((split_kv_kernel<WRV, F8, EV>), grid, dim3(64 * WRV), 0, st, a); \
    return (int)hipGetLastError();                                                   \
  }
  RATTN_VARIANTS(RATTN_LAUNCH)
#undef RATTN_LAUNCH
  return (int)hipErrorInvalidValue;
}

int split_kv_blocks_per_cu(int waves, bool fp8, bool even) {
  const int key = variant_key(waves, fp8, even);
  int nb = 0;
#define RATTN_OCC(WRV, F8, EV)                                                          \
  if (key == variant_key(WRV, F8, EV)) {                                                \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, split_kv_kernel<WRV, F8, EV>, \
                                                        64 * WRV, 0) == hipSuccess ? nb : 0; \
  }
  RATTN_VARIANTS(RATTN_OCC)
#undef RATTN_OCC
  return 0;
}

// The combine's shape for a partition (see combine_kernel): per-unit splits of up to 16
// pieces take whole rows, 8 per work-group; even shares (a few to a few tens of pieces
// per unit) whole rows with 2 stripes, 4 per work-group; per-unit splits of 256 pieces
// or more 16 waves per 32-dim slice; the rest one wave per 32-dim slice.
enum CombineShape { kCombineRows, kCombineRows2, kCombineSlices4, kCombineWide };

static CombineShape combine_shape(int splits_per_unit) {
  if (splits_per_unit == 0) return kCombineRows2;
  if (splits_per_unit <= 16) return kCombineRows;
  if (splits_per_unit >= 256) return kCombineWide;
  return kCombineSlices4;
}

int64_t combine_blocks(int64_t rows, int splits_per_unit) {
  switch (combine_shape(splits_per_unit)) {
    case kCombineRows: return (rows + 7) / 8;
    case kCombineRows2: return (rows + 3) / 4;
    default: return rows * 4;
  }
}

int launch_combine(const KernelArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.batch * a.n * a.num_q_heads;
  const dim3 grid((unsigned)combine_blocks(rows, a.splits_per_unit));
  const hipStream_t st = (hipStream_t)stream;
  switch (combine_shape(a.splits_per_unit)) {
    case kCombineRows:
      hipLaunchKernelGGL((combine_kernel<32, 1, 8, 16>), grid, dim3(256), 0, st, a);
      break;
    case kCombineRows2:
      hipLaunchKernelGGL((combine_kernel<32, 2, 4, 16>), grid, dim3(256), 0, st, a);
      break;
    case kCombineWide:
      hipLaunchKernelGGL((combine_kernel<8, 128, 1, 8>), grid, dim3(1024), 0, st, a);
      break;
    default:
      hipLaunchKernelGGL((combine_kernel<8, 8, 1, 16>), grid, dim3(64), 0, st, a);
      break;
  }
  return (int)hipGetLastError();
}

}  // namespace rattn

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

int launch_append_kv(const AppendArgs& a, void* stream) {
  const int64_t waves = (int64_t)2 * a.batch * a.n * a.num_kv_heads;
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)waves), dim3(64), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rattn
