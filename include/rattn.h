/*
 * rattn -- relative-position GQA decode/verify attention over a paged KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * What one rattn_decode call computes (one attention layer, one decode or verify
 * step): for every sequence b, query row r in [0, n) and query head h,
 *
 *   p   = seq_lens[b] - n + r                 absolute position of row r
 *   g   = h / (num_q_heads / num_kv_heads)    the KV head this query head reads
 *   J   = { j : j <= p  and (window == 0 or p - j <= window - 1) }
 *   s_j = softmax_scale * (q . k_j) + bias[h][min(p - j, dmax)]
 *   out = sum_{j in J} exp(s_j - m) v_j / sum_{j in J} exp(s_j - m),  m = max s_j
 *   lse = m + ln(sum_{j in J} exp(s_j - m))
 *
 * Sources (the text of three web pages on serving the Inkling models with vLLM):
 *   - "vLLM TML Inkling support" (page 2), model architecture section: attention uses
 *     a learned relative-position term added to the logits before the softmax, in
 *     place of rotary embeddings; GQA with head size 128 in every layer; a hybrid of
 *     sliding-window and full-attention layers.
 *   - "vLLM supports Inkling 2 Small" (page 1), model table: 48 query / 8 KV heads,
 *     sliding window 1,024; section on trying the model: 7 speculative tokens per step,
 *     verified by the target model (so up to 8 query rows per sequence, causal among
 *     themselves); section on vLLM's optimisations: a decode kernel that packs the 6
 *     query heads of a GQA group into one tile so K/V are read once per group.
 *   - page 2, technical-optimisation section (FA4 kernel): a "sheared-bias" access
 *     pattern for the relative term, and a split count chosen from batch size and KV
 *     length; roadmap: FP8 global attention. Page 3 ("vLLM supports Reflection Beam"),
 *     support section: an FP8 KV cache; section on coding agents speeding up the
 *     implementation: a chunked prefill (8 x 2048 tokens at about 100K context) and a
 *     fused KV-cache update; section on DFlash2 and adaptive verification: a different
 *     number of verified drafts per sequence.
 * The pages do not fix how the relative term is parameterised; here it is a per-head
 * float32 table indexed by the query-key distance, clamped at dmax.
 *
 * Conventions
 *   - Every tensor pointer is DEVICE memory owned by the caller. A plan owns only its
 *     workspace (split partials), allocated by rattn_plan and released by rattn_free.
 *   - Layouts (row-major, innermost last):
 *       q          bf16  [batch][n][num_q_heads][head_dim]
 *       k_cache    bf16 or E4M3 codes  [num_pages][num_kv_heads][page_size][head_dim]
 *       v_cache    same as k_cache
 *       k_scale    fp32  [num_pages][num_kv_heads][page_size]   (E4M3 cache only)
 *       v_scale    same as k_scale
 *       page_table int32 [batch][max_pages_per_seq]; key j of sequence b is slot
 *                  j % page_size of physical page page_table[b][j / page_size]
 *       seq_lens   int32 [batch]; each length counts the n query rows, whose keys and
 *                  values are already in the cache; n <= seq_lens[b] <= max_seq_len
 *       bias       fp32  [num_q_heads][dmax + 1]
 *       out        bf16  [batch][n][num_q_heads][head_dim]   (round to nearest even)
 *       lse        fp32  [batch][n][num_q_heads], natural log (may be NULL)
 *   - The E4M3 cache holds OCP 8-bit E4M3 ("e4m3fn") codes; the value of a key or value
 *     element is code value * scale of its (page, KV head, slot).
 *   - rattn_decode is asynchronous on `stream` (a hipStream_t; NULL = default stream),
 *     never synchronises the host and allocates nothing, so it can be captured in a HIP
 *     graph. Calls that share a plan share its workspace: use one plan per stream.
 *   - Errors: all calls return a status and never throw across the ABI. Problem and
 *     pointer checks happen on the host before any HIP call (RATTN_E_INVALID,
 *     RATTN_E_UNSUPPORTED). A failed launch returns RATTN_E_HIP; a failed workspace
 *     allocation RATTN_E_NOMEM. Device-side bad data (a length outside [n, max_seq_len],
 *     a page id outside [0, num_pages)) is clamped so nothing is read out of bounds, and
 *     is recorded in a flag word readable with rattn_debug_flags.
 */
#ifndef RATTN_H
#define RATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RATTN_ABI_VERSION 4

typedef struct rattn_plan_s* rattn_plan_t;

typedef enum {
  RATTN_OK = 0,
  RATTN_E_INVALID = 1,      /* a null pointer or an inconsistent problem            */
  RATTN_E_UNSUPPORTED = 2,  /* a valid problem outside what the kernels implement   */
  RATTN_E_HIP = 3,          /* a HIP runtime call or a kernel launch failed          */
  RATTN_E_NOMEM = 4         /* the workspace allocation failed                      */
} rattn_status;

typedef enum {
  RATTN_KV_BF16 = 0,
  RATTN_KV_FP8_E4M3 = 1     /* OCP E4M3 codes plus fp32 per-token-per-head scales   */
} rattn_kv_dtype;

/* Debug flag bits reported by rattn_debug_flags. */
#define RATTN_FLAG_SEQ_LEN_CLAMPED 1   /* a seq_lens entry was outside [n, max_seq_len] */
#define RATTN_FLAG_PAGE_CLAMPED 2      /* a page id was outside [0, num_pages)          */
#define RATTN_FLAG_ROWS_INVALID 4      /* a cu_rows range was not within the row buffers */

typedef struct {
  int32_t batch;             /* sequences, >= 1                                          */
  int32_t num_q_heads;       /* query heads (48 in the Inkling 2 Small layers)            */
  int32_t num_kv_heads;      /* KV heads (8); num_q_heads % num_kv_heads == 0             */
  int32_t head_dim;          /* 128 (the only supported value)                            */
  int32_t n_query_rows;      /* rows per sequence: 1 for decode, 1 + drafts for verify    */
                             /* (up to 9 tokens for MTP steps), the chunk length for a   */
                             /* chunked prefill (see RATTN_KERNEL_PREFILL)               */
  int32_t page_size;         /* slots per page: a power of two >= 16                      */
  int32_t num_pages;         /* physical pages in the cache                               */
  int32_t max_pages_per_seq; /* page_table row length                                     */
  int32_t max_seq_len;       /* upper bound on seq_lens[]; <= max_pages_per_seq*page_size */
  int32_t window;            /* 0 = full context; W > 0 = W keys including the token      */
  int32_t dmax;              /* largest distance with its own bias column (>= 0)          */
  float softmax_scale;       /* multiplies q . k (1/sqrt(head_dim) for the pages' models);*/
                             /* a positive normal float, else RATTN_E_INVALID; the bias  */
                             /* divided by it must stay finite in fp32                   */
  int32_t kv_dtype;          /* rattn_kv_dtype                                            */
  int32_t num_splits;        /* 0 = planner; > 0 forces num_splits pieces (key ranges)    */
                             /* per (sequence, KV head) unit (at most 4096; at most      */
                             /* 65536 in all); 2 or 3 single-wave bf16 pieces run as one */
                             /* work-group per unit (rattn_plan_info.pieces_per_group)   */
} rattn_problem;

typedef struct {
  int32_t num_splits;        /* pieces (key ranges) per (sequence, KV head), nominal      */
  int32_t keys_per_split;    /* keys per piece at max_seq_len, nominal                    */
  int32_t tile_keys;         /* keys per inner-loop step                                  */
  int32_t row_tiles;         /* waves per piece (split: 1, 2, 4 or 8, each with          */
                             /* tiles_per_wave 16-row MFMA tiles; prefill: 8 per group)   */
  int32_t grid_x, grid_y, grid_z;   /* split kernel grid: (work-groups, 1, 1)             */
  int32_t combine_blocks;    /* combine work-groups; 0 when nothing is merged after the   */
                             /* split kernel                                              */
  int32_t num_cus;           /* compute units the plan was sized for                      */
  int32_t blocks_per_cu;     /* resident split-kernel work-groups per CU assumed          */
  int32_t kernel;            /* RATTN_KERNEL_*: which kernel the plan launches            */
  int32_t pieces_per_group;  /* pieces per split work-group, one wave each: 1, or 2 or 3  */
                             /* when a unit is that many single-wave pieces, which one   */
                             /* work-group attends and merges (no combine launch)        */
  int64_t workspace_bytes;   /* partial outputs and log-sum-exps, and a flag word         */
  int32_t tiles_per_wave;    /* 16-row MFMA tiles per split wave: 1, or 3 when one wave    */
                             /* holds all 33-48 packed rows of a piece (full-context      */
                             /* layers over a bf16 cache)                                 */
} rattn_plan_info;

/* rattn_plan_info.kernel. Up to 128 packed rows per (sequence, KV head) (G * n, G =
 * num_q_heads / num_kv_heads; 1, 2, 4 or 8 waves of one 16-row tile each): the split-KV
 * kernel and, when a unit is split, the log-sum-exp combine. More rows (chunked
 * prefill): one MFMA kernel per block of query tokens over all the keys they see, no
 * split; built for G = 4, 6 and 8 over a bf16 cache, without forced splits (else
 * RATTN_E_UNSUPPORTED). */
#define RATTN_KERNEL_SPLIT_KV 0
#define RATTN_KERNEL_PREFILL 1

/* Validate `prob`, size the launch for the current HIP device and allocate the
 * workspace. On success *plan_out owns the workspace until rattn_free.
 * The split of the key range follows page 2 ("vLLM TML Inkling support", technical
 * optimisation section, FA4 kernel): the number of splits is chosen from the batch,
 * the head count and the KV length; here from batch x KV heads, the rows per sequence,
 * the visible key span, the device's compute units and the split kernel's resident
 * work-groups per CU, which this call queries. Problems whose tiles (batch x num_kv_heads
 * x ceil((span + 31) / 32), span = max_seq_len, or window + n - 1 in a window layer)
 * reach 2^31 are RATTN_E_UNSUPPORTED. Allocates device memory (hipMalloc); see
 * rattn_decode for the call itself. */
rattn_status rattn_plan(const rattn_problem* prob, rattn_plan_t* plan_out);

/* Validate `prob` and run the planner for a device with `num_cus` compute units,
 * without touching HIP (host-only; used to inspect and test planner decisions). It
 * assumes the split kernel's gfx950 occupancy (4 resident work-groups per CU), which
 * rattn_plan instead queries from the runtime. */
rattn_status rattn_plan_describe(const rattn_problem* prob, int32_t num_cus,
                                 rattn_plan_info* info);

/* The decisions of an existing plan. */
rattn_status rattn_plan_get_info(rattn_plan_t plan, rattn_plan_info* info);

/* One layer's attention for one decode/verify step (see the top of this file for the
 * arithmetic and the layouts). k_scale / v_scale must be non-NULL exactly for the
 * E4M3 cache; lse may be NULL. */
rattn_status rattn_decode(rattn_plan_t plan, const void* q, const void* k_cache,
                          const void* v_cache, const float* k_scale, const float* v_scale,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const float* bias, void* out, float* lse, void* stream);

/* As rattn_decode, with a different number of query rows per sequence (page 3, "vLLM
 * supports Reflection Beam", section on DFlash2 and adaptive verification: the verifier
 * picks per step which drafts to check; page 2, "vLLM TML Inkling support", model
 * architecture section: up to 9 tokens per step from chained MTP heads). The plan's
 * n_query_rows is the largest row count of a sequence.
 *   cu_rows    device int32 [batch + 1], nondecreasing from cu_rows[0] = 0: sequence b
 *              owns packed rows cu_rows[b] .. cu_rows[b+1]-1, n_b = cu_rows[b+1] -
 *              cu_rows[b] in [0, n_query_rows], which are its last n_b positions (row i
 *              at position L_b - n_b + i; L_b >= n_b)
 *   num_rows   rows that q, out and lse hold (host int; cu_rows[batch] <= num_rows)
 *   q, out     bf16 [num_rows][num_q_heads][head_dim]; lse fp32 [num_rows][num_q_heads]
 * Rows past cu_rows[batch] are not written. A sequence whose range is not within
 * [0, num_rows] or exceeds n_query_rows rows gets no output and sets
 * RATTN_FLAG_ROWS_INVALID; lengths and page ids are checked as for rattn_decode, against
 * n_b. Same plan, workspace and stream rules as rattn_decode. */
rattn_status rattn_decode_varlen(rattn_plan_t plan, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* page_table,
                                 const int32_t* seq_lens, const int32_t* cu_rows,
                                 int32_t num_rows, const float* bias, void* out, float* lse,
                                 void* stream);

/* Write the n newest tokens of every sequence into the paged cache: the step just
 * before rattn_decode (page 3, "vLLM supports Reflection Beam", section on speeding up
 * the implementation: a fused KV-cache update; page 2's roadmap and page 3's support
 * section: an FP8 KV cache). `prob` gives the shapes (batch, n_query_rows = new tokens
 * per sequence, num_kv_heads, page_size, num_pages, max_pages_per_seq, max_seq_len,
 * kv_dtype) and is validated as for rattn_plan; no plan or workspace is needed.
 *   k_new, v_new  bf16 [batch][n][num_kv_heads][head_dim], device
 *   seq_lens      lengths after the step (they count the new tokens); token r of
 *                 sequence b goes to position L_b - n + r, slot (L_b - n + r) % page_size
 *                 of page page_table[b][(L_b - n + r) / page_size]
 *   k_cache ...   as for rattn_decode; written in place
 *   k_scale ...   E4M3 only: the fp32 scale of each written (token, KV head) row
 *   flags         device int32, RATTN_FLAG_* bits OR-ed in for skipped rows (nullable)
 * E4M3 rows: s = max_d |x_d| / 448 (1 for an all-zero row) and codes of clamp(x_d / s,
 * -448, 448) rounded to the nearest E4M3 value (ties to even), the quotients correctly
 * rounded in fp32. A sequence whose length is outside [n, max_seq_len], or a token whose
 * page id is outside [0, num_pages), is not written and sets its flag bit. Asynchronous
 * on `stream`; allocates nothing. */
rattn_status rattn_append_kv(const rattn_problem* prob, const void* k_new, const void* v_new,
                             const int32_t* page_table, const int32_t* seq_lens,
                             void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             int32_t* flags, void* stream);

/* As rattn_decode, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. There is no plan: the
 * call validates `prob` and plans on the host each time (the device's CU count and the
 * split kernel's occupancy are queried once per device and kept), and its split
 * partials, unit records and flag word live in a static device array of 32 MiB that the
 * library's code object gives each GPU it runs on, held until the process ends. The
 * array's address is resolved with hipGetSymbolAddress on the first call on each device
 * (that device current). Nothing is allocated or freed: no hipMalloc, hipFree or
 * allocating library routine.
 *   prob       the problem, as for rattn_plan; a call whose partials would exceed the
 *              array (plan workspace_bytes > 32 MiB, e.g. thousands of forced splits over
 *              many rows) returns RATTN_E_UNSUPPORTED and launches nothing
 *   flags      device int32, RATTN_FLAG_* bits OR-ed in for clamped bad device data (the
 *              caller clears it); NULL = not reported
 *   others     as for rattn_decode (device pointers, layouts, stream)
 * Every call on a GPU shares that GPU's array, which keeps the last call's contents; no
 * part of it needs clearing between calls (every partial is written before the combine
 * reads it). Calls that overlap on one GPU (on two streams, or from two host threads
 * without ordering) race on the array and give wrong results: order them on one stream. */
rattn_status rattn_decode_static(const rattn_problem* prob, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* page_table,
                                 const int32_t* seq_lens, const float* bias, void* out,
                                 float* lse, int32_t* flags, void* stream);

/* Release the plan and its workspace, the split partials that page 2's split-KV
 * design ("vLLM TML Inkling support", FA4 kernel: the key range is split and the splits
 * merged) needs between the split kernel and the combine. NULL is accepted. Frees device
 * memory (hipFree), so no call that uses the plan may still be in flight: synchronise
 * its stream first. Returns RATTN_E_HIP if the runtime reports an error. */
rattn_status rattn_free(rattn_plan_t plan);

/* Read and clear the plan's device flag word (RATTN_FLAG_*). Synchronises `stream`. */
rattn_status rattn_debug_flags(rattn_plan_t plan, int32_t* flags, void* stream);

/* Instrumentation: time the kernels of every `stride`-th rattn_decode (or
 * rattn_decode_varlen) call of this plan (the first call after this one, then every
 * stride-th), for at most `max_calls` calls. Those calls launch their kernels with a
 * pair of HIP events each, which the runtime stamps with the kernel's own start and end
 * (hipExtLaunchKernel), so the durations leave out launch gaps; the other calls are
 * launched as usual. */
rattn_status rattn_profile_begin(rattn_plan_t plan, int32_t max_calls, int32_t stride);

/* Stop recording; waits for the recorded events and writes, per call, the split
 * kernel's and the combine kernel's durations in milliseconds (combine 0 when there
 * is no combine launch). Arrays hold at least max_calls entries; *ncalls receives the
 * number of calls recorded. */
rattn_status rattn_profile_end(rattn_plan_t plan, float* split_ms, float* combine_ms,
                               int32_t* ncalls);

/* Measurement aid (not part of the attention): read `nblocks` blocks of `block_bytes`
 * bytes (a multiple of 1024) of the device buffer `buf`, block order[i] i-th (device int32
 * [nblocks], a permutation of 0..nblocks-1; NULL = in place order; entries outside
 * [0, nblocks) read a clamped block), with the split kernel's load pattern: non-temporal
 * 16-byte loads, each 64-lane pass reading 1 KiB of contiguous bytes, two blocks in flight
 * per wave, `waves` single-wave work-groups sharing the blocks evenly. `sink` is device
 * memory of 1024 bytes that the kernel may write. Asynchronous on `stream`; a benchmark
 * times it to report the read rate this access pattern reaches on the device. */
rattn_status rattn_read_probe(const void* buf, int64_t nblocks, int32_t block_bytes,
                              const int32_t* order, int32_t waves, void* sink, void* stream);

const char* rattn_status_string(rattn_status status);
int32_t rattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RATTN_H */
