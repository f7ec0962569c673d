/*
 * splitkv.h - split-KV partial decode attention for AMD Instinct MI355X (gfx950).
 *
 * Decode-time attention over a paged KV cache is split along each request's KV
 * history into tasks. Every task emits a partial attention state: the output
 * normalised over its own KV subset plus the log-sum-exp (natural log) of its
 * scores (LiquidCP, section 2.1 "Preliminaries"). An exact LSE-weighted merge
 * composes the states into full attention (LiquidCP, section 3, Equation 1;
 * the Helix deep dive, attention step 3: rescale each partial by
 * exp(lse_r - lse_global) and sum). Split counts come from a critical-wave
 * planner (LiquidCP, section 5.2 and appendix A.2).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All functions are extern "C", return an skv_status, and never throw. On a
 *   non-OK status, skv_last_error() returns a thread-local message.
 * - Arguments are validated on the host before anything is enqueued. Device work
 *   is enqueued asynchronously on `stream` (a hipStream_t; NULL = null stream);
 *   no entry point except skv_read_error_flag synchronises.
 * - "host" pointers are CPU memory, "device" pointers are GPU global memory on
 *   the current device. Every device buffer is owned by the caller; the library
 *   allocates no device memory and keeps no device state between calls.
 *
 * Storage formats (all device, row-major, no padding)
 * ---------------------------------------------------
 * T = float (SKV_F32) or bf16 (SKV_BF16); for SKV_FP8_E4M3, q is bf16 and the
 * KV pages hold T = one-byte OCP E4M3 codes. X = 16 / sizeof(T) (4, 8 or 16).
 * q          [total_q][H_q][D]            T; requests concatenated in batch order,
 *                                         request b owning q_lens[b] tokens.
 * GQA keys   [num_pages][H_kv][D/X][P][X] T; 16-byte chunks of X dimensions,
 *                                         tokens of a page adjacent per chunk.
 * GQA values [num_pages][H_kv][D_v][P]    T; per page and head, dimension-major.
 * MLA rows   [num_pages][P][D]            T = bf16 or E4M3, D = 576 (512 latent + 64 rope).
 *                                         The value of a token is the first
 *                                         D_v = 512 entries of its own row, so
 *                                         v_pages must equal k_pages (SPLASH,
 *                                         section 2: KV bytes per token
 *                                         L(d_c + d_r)b; section 3: rows
 *                                         [N_r, H, d_c + d_r], returned width d_c).
 * page_table [batch][max_pages_per_seq]   int32; token j of request b is in page
 *                                         page_table[b][j / P], slot j % P.
 *                                         Entries past ceil(L_b / P) are never read
 *                                         for addressing; slots past L_b in the last
 *                                         page are never consumed.
 * seq_lens   [batch]                      int32; L_b = KV tokens of request b,
 *                                         including its own q_lens[b] new tokens.
 * FP8 scales k_scales, v_scales [num_pages][H_kv] float32 (SKV_FP8_E4M3 only):
 *                                         a stored key is its code's E4M3 value
 *                                         times k_scales[page][kv_head], a value
 *                                         likewise with v_scales (SPLASH,
 *                                         appendix C.1: an FP8 E4M3 KV cache).
 *                                         MLA: one scale per page for the whole
 *                                         row, keys and values alike, so
 *                                         v_scales must equal k_scales.
 * Query token i of request b with n_b tokens sees KV positions
 * [0, L_b - n_b + i] when causal (bottom-right aligned), [0, L_b) otherwise.
 * KV head of query head h is h / (H_q / H_kv).
 *
 * Partial states (plan-defined CSR layout). Request b has s_b splits and
 * rows_b = q_lens[b] * H_q output rows (row = token * H_q + head). State r of
 * request b occupies rows state_row_offset[b] + r * rows_b .. + rows_b - 1 of
 *   o_part   [state_rows][D_v] float32   output normalised over the split's KV
 *   lse_part [state_rows]      float32   natural-log LSE of the split's scores
 * An empty split (no visible KV, possible for causal chunk rows) stores
 * o = 0 and lse = -inf.
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t skv_status;
#define SKV_OK                 0
#define SKV_ERR_INVALID_ARG   -1   /* null pointer, bad size, inconsistent shapes   */
#define SKV_ERR_UNSUPPORTED   -2   /* valid but not implemented (dtype, head dims)  */
#define SKV_ERR_HIP           -3   /* a HIP runtime call or kernel launch failed    */
#define SKV_ERR_NO_MEMORY     -4   /* host allocation failed, or workspace too small */
#define SKV_ERR_PLAN_MISMATCH -5   /* plan built for a different problem description */

/* SKV_FP8_E4M3: bf16 queries; GQA keys and values, or MLA rows, stored as OCP
 * E4M3 bytes with float32 scales per (page, KV head) (skv_decode_attn_partial_fp8). */
typedef enum { SKV_F32 = 0, SKV_BF16 = 1, SKV_FP8_E4M3 = 2 } skv_dtype;

/* Problem description, passed by value in host memory. */
typedef struct skv_attn_desc {
  int32_t batch;              /* B >= 1                                          */
  int32_t num_q_heads;        /* H_q                                             */
  int32_t num_kv_heads;       /* H_kv, divides H_q; MLA: 1                       */
  int32_t head_dim_qk;        /* D: GQA 64 or 128; MLA 576                       */
  int32_t head_dim_v;         /* D_v: GQA == D; MLA 512                          */
  int32_t page_size;          /* P: 16, 32 or 64                                 */
  int32_t max_pages_per_seq;  /* row stride of page_table                        */
  int32_t num_pages;          /* pages in the pool; ids outside [0, num_pages)
                                 are never dereferenced: they set bit 0 of the
                                 device error flag and the task that met one
                                 writes a NaN state (see skv_read_error_flag) */
  int32_t mla;                /* 1: MLA rows (v_pages == k_pages)                 */
  int32_t causal;             /* 1: bottom-right causal rows when q_len > 1      */
  int32_t dtype;              /* skv_dtype of q and the KV pages; SKV_FP8_E4M3
                                 needs a GQA group of 8 or 16 and runs one
                                 query token per task                          */
  float softmax_scale;        /* scores are softmax_scale * <q, k>; must be
                                 positive and finite (SKV_ERR_INVALID_ARG)     */
} skv_attn_desc;

/* Critical-wave model parameters (LiquidCP, section 5.2, Equations 5-6; the
 * pages' H100 calibration is in their Table 2). Model time unit: one KV tile
 * of tile_tokens tokens with all K attention slots busy. */
typedef struct skv_plan_params {
  int32_t tile_tokens;        /* KV tile and split granularity; must be 64       */
  int32_t slots_per_cu;       /* K = num_cu * slots_per_cu; 0 = kernel default   */
  int32_t warps_per_slot;     /* merge waves per slot; 0 = kernel default        */
  int32_t max_splits;         /* upper bound on splits per request (<= 64)       */
  int32_t overlap_reduction;  /* 0: the merge runs after attention (two
                                 launches); 1: the pages' fused engine, where
                                 reduction overlaps the attention tail:
                                 skv_decode_attn then runs attention and merge
                                 in one launch                                   */
  int32_t use_calibration;    /* 1: take rho, delta_attn, delta_red and gamma from
                                 the library's MI355X fit for the kernel the
                                 problem selects (the fields below are ignored) */
  int32_t balanced_candidates; /* 1: the final choice also weighs the
                                 proportional plans whose tasks fit 1-4 waves of
                                 K slots (an addition to the pages' candidates:
                                 NoSplit, the search result, the reference
                                 plan); 0: the pages' candidates only;
                                 -1 (default): the choice measured for the
                                 kernel the problem selects (on for MLA, off
                                 for GQA)                                      */
  int32_t query_tile;         /* query tokens per attention task: 0 (default) =
                                 the kernel's choice (one token, or a tile of
                                 128 / G tokens for bf16 GQA groups of 8 and
                                 16); other values plan that tile size, and a
                                 size the kernel cannot run is refused when
                                 the plan is built (SKV_ERR_UNSUPPORTED)       */
  double rho;                 /* per-tile time floor                             */
  double delta_attn;          /* per attention task overhead, tile-equivalents   */
  double delta_red;           /* per reduction overhead                          */
  double gamma;               /* cost per merged partial vector                  */
  double min_gain;            /* adopt a split plan only if >= this much faster  */
  double tile_time_us;        /* informational: microseconds per model unit      */
} skv_plan_params;

typedef struct skv_plan skv_plan;  /* opaque, immutable, host memory */

typedef struct skv_plan_info {
  int32_t batch;
  int32_t num_tasks;          /* attention work-groups launched                 */
  int32_t total_splits;       /* sum of s_b                                      */
  int32_t slots;              /* K used by the model                             */
  int32_t warps_per_slot;
  int32_t reduction_run;      /* output rows per merge unit                      */
  int32_t num_units;          /* merge units (one wave each)                     */
  int32_t split_adopted;      /* 0: NoSplit kept                                 */
  int64_t state_rows;         /* rows of o_part / lse_part                       */
  int64_t total_rows;         /* rows of the merged output = total_q * H_q       */
  double score;               /* model completion time of the chosen plan        */
  double t_attn;              /* model attention completion of the chosen plan   */
  double nosplit_score;       /* model completion time of NoSplit                */
  double rho, delta_attn, delta_red, gamma;  /* model parameters in effect        */
  double tile_time_us;        /* microseconds per model unit (calibration)       */
  int32_t balanced_candidates; /* 0 or 1: candidate set in effect               */
  int32_t query_tile;         /* query tokens per attention task (consecutive
                                 tokens of one request; the last tile of a
                                 request may hold fewer)                       */
  double reference_score;     /* skv_plan_splits: model completion time of the
                                 reference plan the search started from (its
                                 own or ref_splits); NaN for the other plans   */
} skv_plan_info;

/* Fill p with the library defaults: use_calibration = 1,
 * balanced_candidates = -1, tile 64, max_splits 64, min_gain 0.10, and the
 * pages' Table 2 (H100) values in rho,
 * delta_attn, delta_red and gamma, which apply when use_calibration is 0. */
void skv_plan_params_default(skv_plan_params* p);

/* Critical-wave split plan (LiquidCP, section 5.2 "Plan selection" and
 * "Task ordering"; appendix A.2 "Split planning").
 * desc        host; the problem the plan will be used with.
 * seq_lens    host int32 [batch]; q_lens host int32 [batch] or NULL (all 1).
 * num_cu      compute units of the device (256 on MI355X).
 * n_ext       external states that the merge will add to every row (model cost).
 * params      host or NULL (defaults). ref_splits host int32 [batch] or NULL:
 * out         receives a new plan; release it with skv_plan_destroy.
 * Split boundaries are multiples of tile_tokens; the last split ends at L_b. */
skv_status skv_plan_splits(const skv_attn_desc* desc, const int32_t* seq_lens,
                           const int32_t* q_lens, int32_t num_cu, int32_t n_ext,
                           const skv_plan_params* params, const int32_t* ref_splits,
                           skv_plan** out);

/* Plan with explicit split counts (host int32 [batch], 1 <= s_b <= tiles of b). */
skv_status skv_plan_from_counts(const skv_attn_desc* desc, const int32_t* seq_lens,
                                const int32_t* q_lens, const int32_t* split_counts,
                                int32_t num_cu, int32_t n_ext,
                                const skv_plan_params* params, skv_plan** out);

/* Fixed-chunk plan: request b is split into ceil(L_b / chunk_tokens) pieces
 * [k*c, min((k+1)*c, L_b)); chunk_tokens must be a positive multiple of 64. */
skv_status skv_plan_fixed_chunks(const skv_attn_desc* desc, const int32_t* seq_lens,
                                 const int32_t* q_lens, int32_t chunk_tokens,
                                 int32_t num_cu, skv_plan** out);

skv_status skv_plan_get_info(const skv_plan* plan, skv_plan_info* info);

/* Copy the plan out (host buffers; any may be NULL):
 * split_counts [batch]; split_start / split_end [total_splits] token ranges in
 * request-then-split order; state_row_offset [batch + 1];
 * task_order [num_tasks][4] = (request, kv_head, query tile, split) in the
 * launch order of the attention work-groups. */
skv_status skv_plan_export(const skv_plan* plan, int32_t* split_counts, int32_t* split_start,
                           int32_t* split_end, int64_t* state_row_offset,
                           int32_t* task_order);

/* Bytes of device workspace the plan's descriptors need (a multiple of 256). */
size_t skv_plan_workspace_bytes(const skv_plan* plan);

/* Copy the plan's descriptors into dev_workspace (device, >= workspace bytes)
 * with an asynchronous host-to-device copy on stream, and clear the device
 * error flag it holds. The plan must stay alive until that copy has executed. */
skv_status skv_plan_upload(const skv_plan* plan, void* dev_workspace, size_t bytes,
                           void* stream);

void skv_plan_destroy(skv_plan* plan);

/* Partial attention states for every split of the plan (page-gathered KV
 * streaming, QK^T, online softmax, PV, local normalisation).
 * q, k_pages, v_pages, page_table, seq_lens: device, formats above; seq_lens
 * must hold the values the plan was built from (a task whose request's device
 * length differs reads no KV, writes a NaN state and sets bit 1 of the error
 * flag). workspace: device, uploaded from `plan`. o_part / lse_part: device
 * float32, plan state rows.
 * Kernel choice: bf16 GQA with G = H_q/H_kv of 16 or 8 uses matrix cores (a
 * group of 8 fills the 16 head columns with copies); fp32 GQA and bf16 groups
 * below 8 use vector ALUs; MLA uses matrix cores. */
skv_status skv_decode_attn_partial(const skv_attn_desc* desc, const void* q,
                                   const void* k_pages, const void* v_pages,
                                   const int32_t* page_table, const int32_t* seq_lens,
                                   const skv_plan* plan, const void* workspace,
                                   float* o_part, float* lse_part, void* stream);

/* Exact LSE merge of each row's states (LiquidCP Equation 1): the plan's local
 * splits plus n_ext external states per row (device float32, o_ext
 * [n_ext][total_rows][D_v], lse_ext [n_ext][total_rows]; NULL when n_ext = 0).
 * o_out: device [total_rows][D_v] of out_dtype (float32, or bf16 rounded to
 * nearest even); lse_out: device float32 [total_rows] or NULL.
 * Rows whose states are all empty produce o = 0, lse = -inf; a row with a
 * NaN LSE among its states (a task that met a device error) produces NaN. */
/* FP8 KV cache (SPLASH, appendix C.1, serves an FP8 E4M3 KV cache): as
 * skv_decode_attn_partial for desc->dtype = SKV_FP8_E4M3, with the key and
 * value scales [num_pages][H_kv] float32 (device). Each code is decoded
 * exactly (E4M3 values are bf16 values) and the products run on bf16 matrix
 * cores with fp32 accumulation; the key scale multiplies the block's scores,
 * the value scale its softmax weights. GQA groups of 8 or 16, or MLA rows
 * (v_pages == k_pages and v_scales == k_scales, one scale per page). The other
 * compute entry points reject FP8 descriptions (SKV_ERR_INVALID_ARG);
 * skv_merge_states merges the states as any others. A NaN code yields NaN in
 * the states that read it. */
skv_status skv_decode_attn_partial_fp8(const skv_attn_desc* desc, const void* q, const void* k_pages,
                                       const void* v_pages, const float* k_scales, const float* v_scales,
                                       const int32_t* page_table, const int32_t* seq_lens,
                                       const skv_plan* plan, const void* workspace, float* o_part,
                                       float* lse_part, void* stream);

skv_status skv_merge_states(const skv_attn_desc* desc, const skv_plan* plan,
                            const void* workspace, const float* o_part,
                            const float* lse_part, int32_t n_ext, const float* o_ext,
                            const float* lse_ext, void* o_out, int32_t out_dtype,
                            float* lse_out, void* stream);

/* Bytes of device scratch skv_decode_attn needs for `plan` (a multiple of
 * 256): a 256-byte-aligned block of counters, then the plan's partial states
 * (o_part, lse_part; layouts above). 0 if plan is NULL. */
size_t skv_decode_attn_scratch_bytes(const skv_plan* plan);

/* The whole path in one call: the partial attention state of every split of
 * the plan (as skv_decode_attn_partial) into `scratch`, then their exact merge
 * with n_ext external states into o_out / lse_out (as skv_merge_states), with
 * the same results bit for bit. A plan built with overlap_reduction = 0 runs
 * as those two launches. One built with overlap_reduction = 1 runs as one
 * launch (LiquidCP, section 6.2 and appendix A.3): each work-group computes
 * one task, publishes it through a per-request counter in the scratch, and
 * work-groups that finish after every task has started merge the requests
 * whose tasks have all published. Arguments are those of the two calls;
 * scratch: device, caller-owned, at least skv_decode_attn_scratch_bytes(plan)
 * bytes (SKV_ERR_NO_MEMORY if scratch_bytes is smaller), not read before it
 * is written; the same scratch must not be used by two calls that overlap in
 * time. */
skv_status skv_decode_attn(const skv_attn_desc* desc, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* page_table, const int32_t* seq_lens,
                           const skv_plan* plan, const void* workspace, void* scratch,
                           size_t scratch_bytes, int32_t n_ext, const float* o_ext,
                           const float* lse_ext, void* o_out, int32_t out_dtype, float* lse_out,
                           void* stream);

/* skv_decode_attn over an FP8 E4M3 KV cache (desc->dtype = SKV_FP8_E4M3):
 * the attention as skv_decode_attn_partial_fp8 with its scales, then the
 * merge, through `scratch` as skv_decode_attn. The plan must be built with
 * overlap_reduction = 0 (the two launches; SKV_ERR_UNSUPPORTED otherwise).
 * Arguments, results and errors are otherwise those of the two calls. */
skv_status skv_decode_attn_fp8(const skv_attn_desc* desc, const void* q, const void* k_pages,
                               const void* v_pages, const float* k_scales, const float* v_scales,
                               const int32_t* page_table, const int32_t* seq_lens, const skv_plan* plan,
                               const void* workspace, void* scratch, size_t scratch_bytes, int32_t n_ext,
                               const float* o_ext, const float* lse_ext, void* o_out, int32_t out_dtype,
                               float* lse_out, void* stream);

/* skv_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The scratch is a 128 MiB array in the library's device code: each device
 * that runs this call holds one from the first call on it until the process
 * ends. A plan whose skv_decode_attn_scratch_bytes exceeds 128 MiB gets
 * SKV_ERR_NO_MEMORY before anything else happens. Every call on a device
 * shares that device's array, which keeps the last call's contents: calls
 * that overlap in time on one device (other streams or threads) race and must
 * be serialised by the caller. Arguments, results and errors are otherwise
 * those of skv_decode_attn; no device memory is allocated or freed. */
skv_status skv_decode_attn_noalloc(const skv_attn_desc* desc, const void* q, const void* k_pages,
                                   const void* v_pages, const int32_t* page_table,
                                   const int32_t* seq_lens, const skv_plan* plan,
                                   const void* workspace, int32_t n_ext, const float* o_ext,
                                   const float* lse_ext, void* o_out, int32_t out_dtype,
                                   float* lse_out, void* stream);

/* Synchronise stream and read the workspace's device error flag (bits OR-ed
 * by every launch since the last skv_plan_upload of this workspace):
 * 0 = none;
 * bit 0 (1) = a page id outside [0, num_pages) was met: that id was not
 *             dereferenced and every row of the affected task's partial state
 *             (o_part and lse_part) is NaN, so the merged rows are NaN too;
 * bit 1 (2) = a request's device seq_lens value differs from the plan's: its
 *             tasks read no KV and write NaN states;
 * bit 2 (4) = MLA only: scores whose scaled values fp32 cannot order within
 *             the kernel's two passes (only with absurdly large scales): the
 *             affected state is NaN;
 * bit 3 (8) = one-launch skv_decode_attn only: a merge waited about a second
 *             for its request's tasks and gave up: that request's merged rows
 *             are NaN (not expected; it would mean the launch lost a task).
 * Rows of tasks that met no error are computed normally. */
skv_status skv_read_error_flag(const void* workspace, int32_t* flag, void* stream);

/* Measurement utility (not a step of the method): a streaming read of
 * `bytes` bytes at device address `buf` (16-byte aligned, bytes a positive
 * multiple of 16) with the non-temporal hint, over `blocks` work-groups of
 * 256 threads (1..65536); out: device uint32[blocks], each the XOR of the
 * 32-bit words its work-group read (so the XOR of all of them is the XOR of
 * the buffer). Asynchronous on `stream`; the caller times it. Used to state
 * the practical HBM read ceiling beside the attention kernels' KV streams. */
skv_status skv_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks,
                              void* stream);

/* Measurement utility (not a step of the method): `blocks` work-groups
 * (1..65536) of `waves` waves (1..8). The first `mfma_waves` (0..waves) of
 * each run `iters` (0..2^24) trips of eight independent bf16
 * v_mfma_f32_16x16x32 products on pseudo-random register operands (16384 * 8
 * * iters flop per wave); the others together read the `bytes` bytes at
 * device address `buf` `passes` times (0..1024) with the non-temporal hint
 * (buf 16-byte aligned, bytes a positive multiple of 16; not read, and may be
 * NULL, when mfma_waves == waves). out: device uint32[2 * blocks * waves];
 * for wave w (block-major) out[2w] holds a word folded from its results (the
 * bits of a float sum of its products for a product wave) and out[2w + 1]
 * the shader-clock cycles (s_memtime) of its loop. Asynchronous on `stream`;
 * the caller times it. Used to state the bf16 matrix rate the chip sustains
 * under a dense load, and the rate of a launch that runs nothing but products
 * and an HBM stream in a given proportion: the ceilings of matrix-side
 * attention launches. */
skv_status skv_mfma_probe(const void* buf, int64_t bytes, int32_t passes, uint32_t* out, int32_t blocks,
                          int32_t waves, int32_t mfma_waves, int32_t iters, void* stream);

/* Thread-local message for the last non-OK status of this thread. */
const char* skv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPLITKV_H */
