/*
 * mla_decode.h — C ABI of the MI355X (gfx950) MLA decode library.
 *
 * Multi-head latent attention decode over a paged latent KV cache. For each
 * sequence b, query token s and head h:
 *
 *   n      = ctx_b - S + 1 + s  with the causal mask, else ctx_b
 *   slot_r = kv_page_indices[kv_indptr[b] + r / page_size] * page_size + r % page_size
 *   K_r    = deq(cache[slot_r, 0:576]),  V_r = K_r[0:512]
 *   z_r    = softmax_scale * (q[b,s,h,:] . K_r)          for r < n
 *   out[b,s,h,:] = sum_r exp(z_r - max z) V_r / sum_r exp(z_r - max z)
 *   lse[b,s,h]   = max z + ln(sum_r exp(z_r - max z))
 *
 * deq is exact for bf16 and (fp8 e4m3fn byte value) * kv_scale for fp8.
 *
 * Sources. The pages state no formula; this is the plainest reading of them:
 *  - "HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size + mask support",
 *    Summary: decode over a paged latent cache with a variable page size and a
 *    causal mask for multi-token (MTP) queries; heads x query tokens stacked
 *    into 64- or 128-row tiles; device-side metadata sized for num_cu clusters.
 *  - "[Perf][Kimi-K3] Cut MLA decode concat/cache epilogue latency", Purpose:
 *    the decode FMHA reads the absorbed query (ql_nope joined with q_pe) and
 *    576-wide latent cache rows.
 *  - "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV", description:
 *    KV-chunk grid axis sized from the longest sequence with an early exit for
 *    chunks past a sequence's end; fp8 cache, page size 1.
 * Row layout (latent 512 first, then rope 64), the fp8 flavour (OCP e4m3fn,
 * max 448), the scale 1/sqrt(192) used by the workloads and the split-KV
 * log-sum-exp merge are readings, not statements of the pages.
 *
 * Conventions for every entry point:
 *  - All pointers named d_* are device pointers (HIP device memory of the
 *    current device); everything else is host memory. The caller owns every
 *    buffer; the library never allocates or frees device memory, and never
 *    synchronises the stream (except the mla_debug_* test hooks).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued in call order; the library keeps no state between calls.
 *  - Host-detectable errors are returned before any device work is enqueued.
 *    Device-detectable errors (bad context length, short page list, page
 *    index out of range) set bits in the status word of the workspace; the
 *    kernels clamp every index and never read out of bounds.
 *  - Returns MLA_ERR_HIP if a launch reports an error.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 6
#define MLA_ROW_DIM 576    /* q / cache row width: 512 latent + 64 rope */
#define MLA_LATENT_DIM 512 /* V width = output width */
#define MLA_MAX_SEQLEN_QO 8
#define MLA_PLAN_MAGIC 0x4d4c4132u
#define MLA_SCRATCH_BYTES (96u << 20) /* the static workspace of mla_decode_scratch, per device */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,         /* null pointer, non-positive size, bad enum */
  MLA_ERR_UNSUPPORTED = 2,         /* valid but outside the supported shapes */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < plan->ws_bytes */
  MLA_ERR_HIP = 4,                 /* the HIP runtime reported an error */
  MLA_ERR_BAD_PLAN = 5,            /* plan not made by mla_decode_plan* */
  MLA_ERR_SCRATCH_TOO_SMALL = 6    /* mla_decode_scratch: the call needs more than MLA_SCRATCH_BYTES */
} mla_status_t;

typedef enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3FN = 1 } mla_kv_dtype_t;

/* Query element type. fp8 is the pages' fp8-query x fp8-cache kernel setting
 * ("HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size + mask support",
 * the fp8_fp8 kernels of its file table): each query element is an e4m3fn
 * byte times one per-tensor q_scale. It needs an fp8 cache. */
typedef enum { MLA_Q_BF16 = 0, MLA_Q_FP8_E4M3FN = 1 } mla_q_dtype_t;

/* Status-word bits written to the workspace by the device (word 0 at ws_status_offset). */
#define MLA_DEV_CTX_TOO_SHORT 1u     /* context_lens[b] < seqlen_qo      */
#define MLA_DEV_CTX_TOO_LONG 2u      /* context_lens[b] > max_context_len */
#define MLA_DEV_TOO_FEW_PAGES 4u     /* page list shorter than ceil(ctx/page_size) */
#define MLA_DEV_PAGE_OUT_OF_RANGE 8u /* a page index >= num_slots / page_size (or < 0) */
#define MLA_DEV_STALE_PLAN 16u       /* mla_decode saw context lengths other than the planned ones */

/* Shape and numeric parameters of one decode call. */
typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t seqlen_qo;       /* S, 1..8 query tokens per sequence */
  int32_t num_heads;       /* H >= 1 */
  int32_t page_size;       /* P >= 1 cache rows per page */
  int32_t max_context_len; /* upper bound of context_lens (sizes the chunks and workspace) */
  int32_t causal;          /* 0 or 1: token s sees ctx - S + 1 + s rows */
  int32_t kv_dtype;        /* mla_kv_dtype_t */
  float softmax_scale;     /* multiplies q . k */
  float kv_scale;          /* fp8: per-tensor dequant scale; bf16: must be 1 */
  int64_t num_slots;       /* rows in the cache pool; a multiple of page_size */
  int32_t q_dtype;         /* mla_q_dtype_t; MLA_Q_FP8_E4M3FN needs kv_dtype MLA_KV_FP8_E4M3FN */
  float q_scale;           /* fp8 query: per-tensor dequant scale; bf16 query: must be 1 */
} mla_decode_params_t;

/* Tunables of the work split, per tile class (tile rows 16, 32, 64, 128). */
typedef struct {
  int32_t wg_per_cu[4]; /* persistent workgroups per CU (capped at what the class's kernel holds) */
  int32_t chunk_min[4]; /* chunk length bounds in cache rows, multiples of 64 */
  int32_t chunk_max[4];
  int32_t force_chunk;  /* 0 = use the rule; else this chunk length (multiple of 64) */
} mla_plan_options_t;

/* Host copy of a plan. Made by mla_decode_plan / mla_decode_plan_host; read-only for callers. */
typedef struct {
  uint32_t magic;
  int32_t num_cu;
  mla_decode_params_t params;
  mla_plan_options_t options;
  int32_t heads_per_group; /* hpg = min(H, 128 / S) */
  int32_t num_groups;      /* G = ceil(H / hpg) */
  int32_t rows_per_group;  /* hpg * S valid rows per tile */
  int32_t tile_rows;       /* 16, 32, 64 or 128 */
  int32_t tile_class;      /* log2(tile_rows / 16) */
  int32_t chunk_len;       /* C, cache rows per work item, multiple of 64 */
  int32_t max_chunks;      /* ceil(max_context_len / C) */
  int32_t wg_per_cu;       /* occupancy used: min(options.wg_per_cu[class], what the kernel holds) */
  int32_t num_workgroups;  /* W = num_cu * wg_per_cu: the persistent decode grid */
  int64_t partial_capacity_records; /* B * G * max_chunks */
  int64_t work_capacity;            /* B * max_chunks: entries of the work list */
  uint64_t ws_status_offset;   /* uint32 [4]: status bits, item count, task counter (W between calls), 0 */
  uint64_t ws_nchunks_offset;  /* int32 [B]: chunks of each sequence (0 = invalid sequence) */
  uint64_t ws_partbase_offset; /* int32 [B]: first partial record of each sequence */
  uint64_t ws_part_out_offset; /* float [records][rows_per_group][512]: normalised partial outputs */
  uint64_t ws_part_lse_offset; /* float [records][rows_per_group]: partial lse, base-2 log */
  uint64_t ws_work_offset;     /* int32 [work_capacity][8]: work items, longest first: sequence, chunk, and the
                                  sequence's planned ctx, page-list start, n_b and first record; 0, 0 */
  uint64_t ws_bytes;           /* total workspace bytes needed */
} mla_plan_t;

/* ABI version of the loaded library (MLA_ABI_VERSION). */
int32_t mla_abi_version(void);

/* Human-readable text of a status code (static storage). */
const char* mla_status_string(mla_status_t status);

/* Fills *out with the default tunables: wg_per_cu {1, 1, 2, 1} (the 64-row kernel
 * runs at occupancy 2, as the pages' m16x4 kernel does: "HK MLA: MI35x m16x8
 * retune, new m16x4 kernel, page_size + mask support", Summary);
 * chunk_min {256, 256, 256, 64}, chunk_max {8192, 8192, 4096, 6144}, force_chunk 0. */
void mla_plan_options_default(mla_plan_options_t* out);

/*
 * Host half of the planner: validates params and computes the plan (tile
 * grouping, persistent grid, chunk length, workspace layout) with no device
 * work and no HIP call when num_cu > 0. num_cu <= 0 asks the current device for
 * its CU count. options may be NULL (defaults). Sources: "HK MLA: MI35x m16x8
 * retune, new m16x4 kernel, page_size + mask support", Summary and file table
 * (a persistent decode kernel whose metadata is sized for num_cu clusters,
 * doubled when the 64-row kernel runs at occupancy 2; heads x query tokens
 * stacked into 64- or 128-row tiles) and "perf(mla): chunk the non-FP4
 * gather_kv_b_proj over KV", description (KV chunks sized from the longest
 * sequence, so that few long sequences still fill the device). Rule:
 *   hpg = min(H, 128/S); G = ceil(H/hpg); TR = smallest of 16/32/64/128 >= hpg*S
 *   wg_per_cu = min(options.wg_per_cu[class], fit), fit = workgroups per CU that the
 *               class's decode kernel holds for the cache type (2 for fp8 64-row tiles, else 1)
 *   W = num_cu * wg_per_cu
 *   C = force_chunk or clamp(roundup(ceil(Lmax / want), 64), chunk_min, chunk_max),
 *       want = max(1, floor(W / (B*G)))
 *   max_chunks = ceil(Lmax / C), work_capacity = B * max_chunks
 * Returns MLA_ERR_UNSUPPORTED when the task count B * max_chunks * G or a
 * workspace index would not fit the device's 32-bit arithmetic.
 */
mla_status_t mla_decode_plan_host(const mla_decode_params_t* params, const mla_plan_options_t* options,
                                  int32_t num_cu, mla_plan_t* out_plan);

/* Workspace bytes for a call shape (0 if params or options are invalid). Same
 * rule and sources as mla_decode_plan_host; the caller allocates this many bytes. */
size_t mla_decode_workspace_size(const mla_decode_params_t* params, const mla_plan_options_t* options,
                                 int32_t num_cu);

/*
 * Full planner: the host half above, then one device launch that builds the
 * persistent kernel's metadata ("HK MLA: MI35x m16x8 retune, new m16x4 kernel,
 * page_size + mask support", file table: device-built metadata; "perf(mla):
 * chunk the non-FP4 gather_kv_b_proj over KV", description: KV chunks, none
 * past its sequence's end). Per sequence it validates context_lens[b]
 * (S <= ctx <= max_context_len, enough pages), writes n_b = ceil(ctx_b / C) (0
 * if invalid) and the exclusive prefix sum of partial records; it writes the
 * work list, items (b, chunk) longest first (a scheduling choice of this
 * library): every full chunk (exactly C rows) in (b, chunk) order, then each
 * sequence's partial last chunk (r = ctx - (n_b - 1) C rows) by length class
 * floor(16 r / C), longest class first, ties by b, then (b, -1) for every
 * invalid sequence; and the status words: the bits, the item count, the task
 * counter's start W and a reserved 0. d_context_lens [B] and
 * d_kv_indptr [B+1] are int32 device arrays. The plan holds for the context
 * lengths and page lists it was made with: mla_decode computes with the planned
 * lengths and sets MLA_DEV_STALE_PLAN when d_context_lens differs from them.
 */
mla_status_t mla_decode_plan(const mla_decode_params_t* params, const mla_plan_options_t* options,
                             int32_t num_cu, const int32_t* d_context_lens, const int32_t* d_kv_indptr,
                             void* d_workspace, size_t workspace_bytes, void* stream, mla_plan_t* out_plan);

/*
 * Decode attention over the paged cache ("HK MLA: MI35x m16x8 retune, new m16x4
 * kernel, page_size + mask support", Summary: paged latent cache, any page
 * size, causal mask for multi-token queries, persistent kernel; "[Perf][Kimi-K3]
 * Cut MLA decode concat/cache epilogue latency", Purpose: absorbed query and
 * 576-wide latent rows). A persistent grid of plan->num_workgroups workgroups
 * walks the tasks of the work list: task t is item t / G for head group t % G.
 * Workgroup x first runs task (x mod 8) * (W / 8) + x / 8 when W is a multiple
 * of 8 (x otherwise), then takes the next untaken task from the workspace's
 * task counter (a device-scope atomic) as each task's last block starts, until
 * none is left, so the longest work goes first to whichever workgroup is about
 * to be free; the workgroup that takes the call's last counter value sets the
 * counter back to W for the next call. Calls sharing one workspace must not
 * overlap (stream-order them).
 *   d_q              [B, S, H, 576], contiguous: bf16, or e4m3fn bytes (value = byte * q_scale)
 *                    when params.q_dtype is MLA_Q_FP8_E4M3FN
 *   d_kv_cache       [num_slots, 576] bf16 or fp8 e4m3fn bytes, contiguous
 *   d_kv_indptr      int32 [B+1]: page list of b is d_kv_page_indices[indptr[b] .. indptr[b+1])
 *   d_kv_page_indices int32 page ids (page p holds slots p*P .. p*P+P-1)
 *   d_context_lens   int32 [B]: compared with the planned lengths, which the call uses
 *                    (MLA_DEV_STALE_PLAN when they differ)
 *   d_out            bf16 [B, S, H, 512]: written for sequences with n_b == 1;
 *                    sequences with n_b > 1 are written by mla_split_combine;
 *                    invalid sequences are filled with NaN
 *   d_lse            float [B, S, H] natural-log lse, or NULL
 *   d_workspace      the workspace given to mla_decode_plan
 */
mla_status_t mla_decode(const mla_plan_t* plan, const void* d_q, const void* d_kv_cache,
                        const int32_t* d_kv_indptr, const int32_t* d_kv_page_indices,
                        const int32_t* d_context_lens, void* d_out, float* d_lse, void* d_workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Log-sum-exp merge of split-KV partials: for every (b, s, h) of a sequence
 * with n_b > 1, with M = max_c lse_c and w_c = 2^(lse_c - M) (partials hold
 * base-2 lse), out = bf16(sum_c w_c o_c / sum_c w_c) and lse = (M + log2 sum_c w_c) * ln 2.
 * Partials with lse = -inf (no visible rows) weigh 0. The pages describe no
 * merge; this is the standard identity for a softmax split over disjoint rows.
 * Sequences with n_b <= 1 are left untouched.
 */
mla_status_t mla_split_combine(const mla_plan_t* plan, void* d_workspace, size_t workspace_bytes,
                               void* d_out, float* d_lse, void* stream);

/*
 * Test hook: synchronously copies the planner's device arrays to host memory
 * (any pointer may be NULL). h_nchunks and h_partbase hold B int32 each,
 * h_status the 4 status words.
 */
mla_status_t mla_debug_read_plan_arrays(const mla_plan_t* plan, const void* d_workspace, int32_t* h_nchunks,
                                        int32_t* h_partbase, uint32_t* h_status);

/*
 * Test hook: synchronously copies the work list to host memory. *h_count
 * receives the number of items; h_items (may be NULL) receives 8 * count
 * int32 (the items, as in ws_work_offset) and must hold 8 * plan->work_capacity.
 */
mla_status_t mla_debug_read_work_list(const mla_plan_t* plan, const void* d_workspace, int32_t* h_count,
                                      int32_t* h_items);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The same work as
 * mla_decode_plan + mla_decode + mla_split_combine on the caller's buffers, with
 * the workspace in a static device array of MLA_SCRATCH_BYTES held by each
 * device that loads the library until the process ends. Calls no hipMalloc,
 * hipFree or allocating routine; the first call on a device looks up that
 * device's array once. A call whose workspace (mla_decode_workspace_size) is
 * larger than MLA_SCRATCH_BYTES returns MLA_ERR_SCRATCH_TOO_SMALL before any
 * device work; use the workspace entry points for it. Every call on one device
 * shares that device's array: the planner rewrites everything the decode reads,
 * so nothing from an earlier call needs clearing, but calls that overlap on one
 * device (unordered streams, or other host threads) race and must not be made.
 * Arguments as for mla_decode_plan and mla_decode; out_plan (may be NULL)
 * receives the plan, whose workspace offsets are into that array.
 */
mla_status_t mla_decode_scratch(const mla_decode_params_t* params, const mla_plan_options_t* options,
                                int32_t num_cu, const void* d_q, const void* d_kv_cache, const int32_t* d_kv_indptr,
                                const int32_t* d_kv_page_indices, const int32_t* d_context_lens, void* d_out,
                                float* d_lse, void* stream, mla_plan_t* out_plan);

/* ---- decode epilogue: query concat and latent-cache insert ---------------- */

/* Bits mla_qcat_cache_insert may set in *d_status. */
#define MLA_INSERT_SLOT_OUT_OF_RANGE 1u     /* slot_mapping[t] >= num_slots: that cache row is not written */
#define MLA_INSERT_POSITION_OUT_OF_RANGE 2u /* positions[t] outside the rope table: not written either */

typedef struct {
  int32_t num_tokens;     /* T >= 0 */
  int32_t num_heads;      /* H >= 1 query heads per token */
  int32_t kv_dtype;       /* mla_kv_dtype_t of the cache */
  float kv_scale;         /* fp8: stored = e4m3fn(value / kv_scale); bf16: must be 1 */
  int64_t num_slots;      /* rows of the cache */
  int32_t rope_positions; /* rows of the cos/sin table */
  int32_t rope_neox;      /* 0: rope pairs (2i, 2i+1); 1: pairs (i, i + 32) */
} mla_insert_params_t;

/*
 * The epilogue that produces mla_decode's inputs ("[Perf][Kimi-K3] Cut MLA
 * decode concat/cache epilogue latency", Purpose: one fused kernel between the
 * absorbed-query GEMM and decode attention, rows (token, head + 1)). For every
 * token t:
 *   q[t, h, 0:512] = ql_nope[t, h] and q[t, h, 512:576] = q_pe[t, h] (bit copy);
 *   if slot_mapping[t] >= 0: cache row slot_mapping[t] = kv_c[t] | rope(k_pe[t]).
 * Rope rotates 32 pairs, (2i, 2i+1) or with rope_neox (i, i + 32), by
 * c = cos_sin[pos][i], s = cos_sin[pos][32 + i] with pos = positions[t]:
 * x' = x c - y s, y' = y c + x s, float32 products then a float32 sum (no fused
 * multiply-add). bf16 cache: round to nearest even; fp8 cache: e4m3fn of
 * value / kv_scale (float32 division), saturated to +-448, nearest even, NaN
 * -> 0x7f. The page prints no per-element arithmetic: these are this library's
 * readings. One lane moves 16 bytes of a 576-wide row, 72 lanes per row.
 *   d_ql_nope bf16 [T, H, 512]   d_q_pe bf16 [T, H, 64]   d_kv_c bf16 [T, 512]
 *   d_k_pe bf16 [T, 64]          d_positions int32 [T]    d_cos_sin float [rope_positions, 64]
 *   d_slot_mapping int64 [T]     d_q bf16 [T, H, 576]     d_cache [num_slots, 576] bf16 or fp8
 *   d_status uint32 or NULL: MLA_INSERT_* bits are OR-ed in
 * Every buffer is contiguous, 16-byte aligned and owned by the caller.
 * Host-detectable errors return before any device work; T = 0 does nothing.
 */
mla_status_t mla_qcat_cache_insert(const mla_insert_params_t* params, const void* d_ql_nope, const void* d_q_pe,
                                   const void* d_kv_c, const void* d_k_pe, const int32_t* d_positions,
                                   const float* d_cos_sin, const int64_t* d_slot_mapping, void* d_q, void* d_cache,
                                   uint32_t* d_status, void* stream);

/* ---- cached-prefix expansion: gather + kv_b_proj --------------------------- */

/* Bits mla_gather_kv_b_proj may set in *d_status. */
#define MLA_KVB_TOO_FEW_PAGES 1u      /* a row's page is past the sequence's page list: row read as zeros */
#define MLA_KVB_SLOT_OUT_OF_RANGE 2u  /* a page id puts the row outside the cache: row read as zeros */
#define MLA_KVB_ROWS_OUT_OF_RANGE 4u  /* cu_ctx[b] < 0, decreasing, or past num_out_rows: sequence not written */
#define MLA_KVB_CTX_TOO_LONG 8u       /* a sequence is longer than max_context_len: rows past it not written */

typedef struct {
  int32_t batch;           /* B >= 0 sequences */
  int32_t num_heads;       /* H >= 1 (local) heads of the projection */
  int32_t page_size;       /* >= 1 cache rows per page */
  int32_t kv_dtype;        /* mla_kv_dtype_t of the cache */
  float kv_scale;          /* fp8: value = e4m3fn byte value * kv_scale; bf16: must be 1 */
  int32_t max_context_len; /* >= every ctx_b; sizes the KV-chunk axis of the launch */
  int64_t num_slots;       /* rows of the cache */
  int64_t num_out_rows;    /* rows of d_k_out and d_v_out (>= cu_ctx[B]) */
} mla_kv_b_proj_params_t;

/*
 * Expands the cached prefix of every sequence from the paged latent into full
 * per-head K and V ("perf(mla): chunk the non-FP4 gather_kv_b_proj over KV",
 * description: one program per (batch, head, KV chunk), chunks past a
 * sequence's end exit at once). Sequence b has ctx_b = cu_ctx[b+1] - cu_ctx[b]
 * cached rows; row r < ctx_b is cache slot
 * kv_page_indices[kv_indptr[b] + r / page_size] * page_size + r % page_size,
 * c = its first 512 values (times kv_scale for fp8), k_pe its last 64. For
 * output row o = cu_ctx[b] + r and head h:
 *   k[o, h, 0:128]   = W[h][0:128]   . c     (float32 accumulation, bf16 round to nearest even)
 *   k[o, h, 128:192] = k_pe                  (bf16: bit copy; fp8: bf16(float(e4m3fn) * kv_scale))
 *   v[o, h, 0:128]   = W[h][128:256] . c
 * The page prints no formula: the reading is the standard MLA up-projection
 * with W laid out as [H * 256, 512] (per head 128 K rows then 128 V rows).
 *   d_kv_cache [num_slots, 576] bf16 or fp8   d_kv_indptr int32 [B + 1]
 *   d_kv_page_indices int32 [kv_indptr[B]]     d_cu_ctx int32 [B + 1], cu_ctx[0] = 0 normally
 *   d_w_kv_b bf16 [H, 256, 512]                d_k_out bf16 [num_out_rows, H, 192]
 *   d_v_out bf16 [num_out_rows, H, 128]        d_status uint32 or NULL: MLA_KVB_* bits are OR-ed in
 * Output rows that belong to no sequence are left untouched. Every buffer is
 * contiguous, 16-byte aligned and owned by the caller. Host-detectable errors
 * return before any device work; B = 0 or max_context_len = 0 does nothing;
 * MLA_ERR_UNSUPPORTED when B * ceil(max_context_len / 256) * H >= 2^31 (the
 * programs of 256 cached rows and one head are counted in 32 bits).
 */
mla_status_t mla_gather_kv_b_proj(const mla_kv_b_proj_params_t* params, const void* d_kv_cache,
                                  const int32_t* d_kv_indptr, const int32_t* d_kv_page_indices,
                                  const int32_t* d_cu_ctx, const void* d_w_kv_b, void* d_k_out, void* d_v_out,
                                  uint32_t* d_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
