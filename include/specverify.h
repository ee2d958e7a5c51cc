/*
 * specverify.h -- C ABI of libspecverify: batched lossless verification of
 * speculative-decoding drafts and the batch-shared verification budget, on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the AngelSpec pages:
 *  - "AngelSpec: specialize the drafter, share the verification budget"
 *    (ai.thesatyajit.com): intro (the target verifies every draft in one pass
 *    and only emits what it would have sampled), section "MTP: fix position 2
 *    and 3" (equation L_e2e: one rejection invalidates every later position,
 *    so accepted length is a sum of prefix products of acceptance rates),
 *    section "D-cut" (Figure 3, equations A-hat and K_rho: prefix-confidence
 *    products, flattened over the batch, global top-K).
 *  - "Tencent open-sources AngelSpec" (tradepoint.io): section "Why one
 *    universal drafter underperforms" (lossless rejection sampling in one
 *    target forward), section "The MTP path" (greedy T = 0 results, MAL).
 * The accept rule u < min(1, p/q), the correction draw from
 * normalize(max(0, p - q)) and the bonus draw from p are the standard
 * speculative-sampling rule that the pages call lossless rejection sampling.
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls (the one exception
 *    is the static scratch array of sv_verify_batch_noalloc).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous and stream-ordered; the library never synchronises the
 *    host.  Results are ready when the stream reaches them.
 *  - Host-checkable argument problems return an error status before any GPU
 *    work is queued (nothing is written).  Launch failures return
 *    SV_ERR_DEVICE.  Problems that only the data reveal (a NaN row, a token
 *    id out of range) are reported per request in sv_diag.bits, with that
 *    request's outputs set to "nothing emitted".
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
  SV_OK = 0,
  SV_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, negative size, D_max > 64 ... */
  SV_ERR_UNSUPPORTED = 2,        /* misaligned rows, unknown dtype or flag         */
  SV_ERR_WORKSPACE_TOO_SMALL = 3,
  SV_ERR_DEVICE = 4,             /* a HIP launch failed                            */
  SV_ERR_SCRATCH_TOO_SMALL = 5   /* sv_verify_batch_noalloc: the batch needs more
                                    than SV_NOALLOC_SCRATCH_BYTES of scratch        */
} sv_status;

typedef enum sv_dtype { SV_DTYPE_BF16 = 0, SV_DTYPE_FP32 = 1 } sv_dtype;

/* Largest draft depth per request (the first-rejection scan is one 64-lane
 * wavefront ballot). */
#define SV_MAX_DEPTH 64
/* Largest B * D_max the single-workgroup budget sort accepts. */
#define SV_MAX_BUDGET_POSITIONS 4096
/* Most vocabulary shards of sv_verify_batch_sharded. */
#define SV_MAX_SHARDS 16

/* Number of stage events sv_verify_batch records when asked to. */
#define SV_NUM_STAGE_EVENTS 5

/* sv_verify_args.flags */
#define SV_FLAG_FORCE_FP64_DRAW 1u /* take every T > 0 draw on the float64 path */
#define SV_FLAG_STREAMING_ROW_PASS 2u /* use the streaming row pass (two reads of each row
                                         pair) instead of the register-resident team pass */
#define SV_FLAG_EXACT_FP64_MASSES 4u  /* float64 draws: compute every tile mass directly
                                         with the float64 normalisers (a second pass over the
                                         row) instead of from the one-pass decomposition */
#define SV_FLAG_TEAM_WAIT_GIVE_UP 8u  /* testing: every team wait of the team row pass gives
                                         up at once, so every member takes the fallback
                                         (streams the pair's full rows itself); results are
                                         those of a normal call, only slower */

/* sv_diag.bits */
#define SV_BIT_BAD_DEPTH 1u        /* depth[r] outside [0, D_max]                      */
#define SV_BIT_BAD_TOKEN 2u        /* a draft token outside [0, V)                     */
#define SV_BIT_BAD_ROW 4u          /* a verified row has NaN / +inf or is all -inf     */
#define SV_BIT_RESIDUAL_ZERO 8u    /* residual mass was zero: the draw used p          */
#define SV_BIT_BAD_TEMPERATURE 16u /* temperature[r] negative, NaN or infinite, or T > 0
                                      so small that a verified row's maximum m gives
                                      |m * (log2(e) / T)| >= 2^24 in float32, past the
                                      exact range of the row-state arithmetic (below
                                      T ~ 1e-5 for logits near 100; use T = 0) */
#define SV_BIT_FP64_DRAW 32u       /* the draw was recomputed in float64               */
#define SV_BIT_SYNC_TIMEOUT 64u    /* information only: a team wait of the row pass
                                      expired (members of a team were not resident at
                                      once, e.g. other work held compute units) and the
                                      waiting member took its row normalisers from the
                                      full rows itself; results are valid */

/* Per-request diagnostics (written when sv_verify_args.diag != NULL). */
typedef struct sv_diag {
  float accept_margin; /* min over tested positions of |u - p(d)/q(d)| (T > 0), else +inf */
  float draw_margin;   /* distance of u*R to the nearest CDF boundary of the draw (T > 0) */
  uint32_t bits;       /* SV_BIT_* */
  int32_t reserved;
} sv_diag;

/* Human-readable name of a status code (static string). */
const char* sv_status_string(sv_status status);

/* Library version string (static). */
const char* sv_version(void);

/* K_rho(B) = max(B, ceil(rho * B * (D + 1))): the verification budget of
 * equation K_rho ("AngelSpec: specialize the drafter...", section "D-cut").
 * Returns -1 for B < 0, D < 0 or rho outside [0, 1]. */
int64_t sv_k_rho(int32_t B, int32_t D, double rho);

/* ---------------------------------------------------------------------------
 * sv_allocate_budget -- the D-cut budget ("AngelSpec: specialize the
 * drafter...", section "D-cut", Figure 3 and equation A-hat).
 *
 * For request r and draft position k (0-based) the score is the prefix
 * confidence product s[r][k] = c[r][0] * c[r][1] * ... * c[r][k], multiplied
 * left to right in float32 (confidences are clamped to [0, 1], NaN reads as
 * 0).  All (r, k < max_depth[r]) are ranked by score, ties by lower r then
 * lower k, and the first K are kept (K clamped to [0, sum max_depth]).  Since
 * scores never increase along a request, each request keeps a prefix:
 *   depth[r]       = number of kept positions of r,
 *   draft_row0[r]  = sum_{i<r} depth[i]         (packed draft rows),
 *   target_row0[r] = sum_{i<r} (depth[i] + 1)   (packed target rows: the
 *                    kept positions plus the bonus row).
 * utility (optional, float[2]) = (sum of kept scores, sum of all scores).
 *
 * conf: float [B, D_max] row-major.  max_depth: int32 [B] or NULL (= D_max).
 * Requires B >= 0, D_max >= 0, B * D_max <= SV_MAX_BUDGET_POSITIONS.
 * ------------------------------------------------------------------------- */
sv_status sv_allocate_budget(const float* conf, int32_t B, int32_t D_max,
                             const int32_t* max_depth, int64_t K, int32_t* depth,
                             int64_t* draft_row0, int64_t* target_row0, float* utility,
                             void* stream);

/* ---------------------------------------------------------------------------
 * sv_allocate_fixed_depth -- the fixed-depth baseline that the budget widget
 * of "AngelSpec: specialize the drafter...", section "D-cut", sets against
 * the global top-K: the same K draft positions spread evenly, every request
 * cut at depth floor(K / B) and the first K mod B requests one deeper, never
 * past D_max (K < 0 reads as 0).  depth, draft_row0, target_row0 as
 * sv_allocate_budget writes them; utility (optional, float[2]) = (sum of the
 * kept positions' prefix-confidence products, sum over all B * D_max
 * positions), products as in sv_allocate_budget, so that
 * utility[0] / utility[1] of the two calls at one K is the widget's retained
 * utility, fixed vs global.  Same size limits and errors as
 * sv_allocate_budget.
 * ------------------------------------------------------------------------- */
sv_status sv_allocate_fixed_depth(const float* conf, int32_t B, int32_t D_max, int64_t K,
                                  int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                                  float* utility, void* stream);

/* ---------------------------------------------------------------------------
 * sv_verify_batch -- lossless verification of a batch of drafted blocks
 * (tradepoint.io page, "Why one universal drafter underperforms": the target
 * verifies the drafts in one pass with rejection sampling; "AngelSpec:
 * specialize the drafter...", section "MTP": one rejection invalidates every
 * later position).
 *
 * Request r has n = depth[r] draft tokens d_k = draft_tokens[r * D_max + k]
 * (k < n), target rows target_row0[r] + k for k = 0..n (row n scores the
 * token after the block: the bonus row) and draft rows draft_row0[r] + k for
 * k < n.  Row i of a logits buffer starts at element i * row_stride.  With
 * s = 1 / temperature[r], p_k = softmax(s * target row k),
 * q_k = softmax(s * draft row k) over all V entries (-inf entries are
 * masked tokens).
 *
 * T > 0: position k keeps d_k if u_k < p_k(d_k) / q_k(d_k), where
 *   (w0, w1, w2, w3) = Philox4x32-10(key = (seed low, seed high),
 *                                    counter = (k, request_id[r], step, 0))
 *   and u_k = (w0 >> 8) * 2^-24.  tau = first rejected position, or n.
 *   If tau < n the token emitted at tau is drawn from normalize(max(0, p - q))
 *   of position tau, else from p_n (the bonus row); the draw takes the
 *   smallest y whose cumulative mass exceeds u' * R, u' = (w1 >> 8) * 2^-24
 *   of counter (tau, ...), R the total mass.  The draw is computed in
 *   float32 and recomputed in float64 whenever the float32 distance to a CDF
 *   boundary is below 1e-5.
 * T = 0: position k keeps d_k if d_k == argmax p_k (lowest index on ties);
 *   the token at tau is argmax of target row tau.  Draft rows are not read
 *   (draft_logits may be NULL when every temperature is 0).
 *
 * Outputs: accepted_len[r] = tau; out_tokens[r * (D_max + 1) + i] = d_i for
 * i < tau, the drawn token at i = tau, -1 after; num_out[r] = tau + 1.
 * alpha (optional, float [B, D_max]): the acceptance rate
 * sum_y min(p_k(y), q_k(y)) = 1 - TV(p_k, q_k) of every k < n (at T = 0:
 * 1 if d_k == argmax p_k else 0); 0 for k >= n.  diag (optional, [B]).
 * An invalid request (see SV_BIT_*) gets accepted_len 0, num_out 0 and
 * out_tokens all -1.
 *
 * Layout requirements: logits base pointers 16-byte aligned and row_stride
 * a multiple of 8 elements (bf16) / 4 elements (fp32), row_stride >= V;
 * 1 <= V < 2^31; 0 <= D_max <= SV_MAX_DEPTH; B (D_max + 1) <= (2^31 - 1) / 64
 * and B ceil(V / 2048) < 2^31 (SV_ERR_INVALID_ARGUMENT otherwise); row
 * indices must address rows inside the caller's buffers.  workspace: device memory of at least
 * sv_verify_workspace_bytes(B, D_max, V) bytes, 256-byte aligned; its
 * contents need no initialisation and are scratch after the call.
 * ------------------------------------------------------------------------- */
typedef struct sv_verify_args {
  sv_dtype dtype;
  int32_t B;
  int32_t D_max;
  int32_t reserved0;
  int64_t V;
  int64_t row_stride;
  const void* target_logits;
  const int64_t* target_row0;  /* [B] */
  const void* draft_logits;
  const int64_t* draft_row0;   /* [B]; may be NULL when every temperature is 0 */
  const int32_t* draft_tokens; /* [B, D_max] */
  const int32_t* depth;        /* [B] */
  const float* temperature;    /* [B] */
  const uint32_t* request_id;  /* [B] or NULL: request_id = r */
  uint64_t seed;
  uint32_t step;
  uint32_t flags;              /* SV_FLAG_* */
  int32_t* accepted_len;       /* [B] */
  int32_t* out_tokens;         /* [B, D_max + 1] */
  int32_t* num_out;            /* [B] */
  float* alpha;                /* [B, D_max] or NULL */
  sv_diag* diag;               /* [B] or NULL */
  void* workspace;
  size_t workspace_bytes;
  /* NULL, or SV_NUM_STAGE_EVENTS hipEvent_t handles (created by the caller)
   * that are recorded on `stream` at the stage boundaries: [0] before the
   * work-list planner, [1] after it, [2] after the row pass (row statistics
   * and acceptance rates), [3] after the accept scan, [4] after the draw.
   * An entry may be NULL (not recorded).  For timing only. */
  void* const* stage_events;
  /* Acceptance statistics of this batch, each optional (NULL: not written):
   * exactly what sv_accept_stats(depth, alpha, accepted_len, B, D_max,
   * stats_expected_len, stats_per_depth, stats_summary) would write after
   * the call returns, the same bits, without a launch of their own (one
   * extra workgroup of the last verification kernel computes them).  Sizes
   * [B], [3 * D_max] and [4] floats on the device; see sv_accept_stats. */
  float* stats_expected_len;
  float* stats_per_depth;
  float* stats_summary;
} sv_verify_args;

/* ---------------------------------------------------------------------------
 * sv_verify_batch_sharded -- the same verification with the vocabulary split
 * over n_shards buffers, as a tensor-parallel target leaves its logits (the
 * pages' target runs with TP = 8: "AngelSpec: specialize the drafter...",
 * section "The numbers"); here every shard sits on the one GPU.
 *
 * Shard s holds columns [s * shard_width, min(V, (s + 1) * shard_width)) of
 * every target row in target_shards[s] and of every draft row in
 * draft_shards[s] (NULL array: no draft logits, as draft_logits = NULL),
 * all with row stride args->row_stride (>= shard_width).  n_shards must equal
 * ceil(V / shard_width), 1 <= n_shards <= SV_MAX_SHARDS, shard_width a
 * multiple of 8 elements, every shard pointer 16-byte aligned.
 * args->target_logits and args->draft_logits are ignored; everything else,
 * the outputs and the workspace are as for sv_verify_batch, and so are the
 * results: the method is that of the concatenated rows.  The team row pass
 * tiles the concatenated row exactly as an unsharded one (a member's slice
 * may span two shards; each 16-byte vector lies in one, its address resolved
 * once per thread), so the row normalisers are the associative (max, sum)
 * merge of slice states and sum min(p, q) a sum of slice sums; the draw scans
 * tile masses in column order across shards.  SV_ERR_UNSUPPORTED when a row
 * needs more team members than fit (no streaming fallback here) or for a
 * shard width that is not a multiple of 8.
 * ------------------------------------------------------------------------- */
sv_status sv_verify_batch_sharded(const sv_verify_args* args, int32_t n_shards,
                                  int64_t shard_width, const void* const* target_shards,
                                  const void* const* draft_shards, void* stream);

/* Device scratch needed by sv_verify_batch for these sizes (0 on bad sizes). */
size_t sv_verify_workspace_bytes(int32_t B, int32_t D_max, int64_t V);

sv_status sv_verify_batch(const sv_verify_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * sv_verify_batch_noalloc -- sv_verify_batch for callers that cannot
 * allocate device memory at all (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same verification, the same
 * kernels and the same results, with the scratch taken from a static device
 * array of SV_NOALLOC_SCRATCH_BYTES that the library holds on each device
 * until the process ends, instead of the caller's workspace.
 *
 * args->workspace and args->workspace_bytes are ignored; every other field,
 * the outputs and the errors are those of sv_verify_batch.  A batch whose
 * sv_verify_workspace_bytes(B, D_max, V) exceeds SV_NOALLOC_SCRATCH_BYTES is
 * rejected with SV_ERR_SCRATCH_TOO_SMALL before any GPU work (32 MiB covers
 * D_max = 16 up to B = 354 requests at V = 262144 and up to B = 426 at
 * V = 151936).  The call allocates nothing: no hipMalloc, no hipFree and
 * no allocating library routine.  The first call on a device resolves the
 * array's device address there (hipGetSymbolAddress, with that device
 * current), which also loads the library's code object on that device if no
 * earlier call did.
 *
 * Every call on one device uses that device's one array, and the scratch
 * holds the last call's contents (the kernels clear what must start at zero
 * themselves).  Calls that overlap on one device -- on different streams, or
 * from different host threads without ordering -- race on the array and give
 * undefined results; order them on one stream.
 * ------------------------------------------------------------------------- */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)

sv_status sv_verify_batch_noalloc(const sv_verify_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * sv_accept_stats -- acceptance statistics of one verified batch (equation
 * L_e2e of "AngelSpec: specialize the drafter...", section "MTP", and the
 * MAL / mean-acceptance figures of the tradepoint.io page, "The MTP path",
 * which satisfy MAL = 1 + D * mean acceptance).
 *
 * Inputs (device): depth[B] (n_r, clamped to [0, D_max]), alpha[B, D_max]
 * (may be NULL), accepted_len[B].
 * Outputs (device float, each optional):
 *   expected_len[B]    E[tau_r] = sum_{m < n_r} prod_{k <= m} alpha[r][k]
 *   per_depth[3*D_max] #requests that tested position k, #that kept it,
 *                      mean alpha at k over requests with depth > k
 *   summary[4]         (mean(tau + 1), 1 + mean E[tau], sum tau / sum n, sum n)
 * ------------------------------------------------------------------------- */
sv_status sv_accept_stats(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                          int32_t B, int32_t D_max, float* expected_len, float* per_depth,
                          float* summary, void* stream);

/* ---------------------------------------------------------------------------
 * sv_accept_stats_accumulate -- statistics over many verified batches, e.g.
 * the steps of a decode loop: MAL, mean acceptance and position-wise
 * acceptance over whole generations, as the tradepoint.io page, "The MTP
 * path", reports them (MAL 2.58 -> 2.99 with mean acceptance 52.8% -> 66.4%
 * at depth 3; position-1 acceptance 0.799 -> 0.814).
 *
 * Adds one batch to the caller's running totals accum (device double
 * [3 + 2 * D_max], zeroed by the caller before the first batch):
 *   accum[0] += sum_r (tau_r + 1)        tokens emitted
 *   accum[1] += B                        requests
 *   accum[2] += sum_r E[tau_r]           (alpha given; equation L_e2e)
 *   accum[3 + k] += #{r: depth_r > k}    position k + 1 verified
 *   accum[3 + D_max + k] += #{r: tau_r > k}  position k + 1 accepted
 * (depth clamped to [0, D_max]; counts are exact integers in double up to
 * 2^53), then writes summary (device float [3 + D_max], optional) from the
 * new totals: [0] MAL = accum[0] / accum[1], [1] expected MAL
 * 1 + accum[2] / accum[1], [2] mean acceptance sum tau / sum depth, [3 + k]
 * position-wise acceptance P(tau >= k + 1) = accum[3 + D_max + k] /
 * accum[1].  With every depth equal to D_max, MAL = 1 + D_max * mean
 * acceptance = 1 + sum of the position-wise acceptances.
 * Inputs: depth [B], accepted_len [B] (device int32), alpha [B, D_max]
 * (device float) or NULL.  Stream-ordered; one call at a time per accum.
 * ------------------------------------------------------------------------- */
sv_status sv_accept_stats_accumulate(const int32_t* depth, const float* alpha,
                                     const int32_t* accepted_len, int32_t B, int32_t D_max,
                                     double* accum, float* summary, void* stream);

/* ---------------------------------------------------------------------------
 * sv_draft_confidence -- the drafter's confidence in each drafted token, the
 * scores the D-cut budget ranks ("AngelSpec: specialize the drafter...",
 * section "D-cut": Figure 3 panel 1, confidence-scored candidate tokens;
 * equation A-hat multiplies them along a request).
 *
 * conf[r * D_max + k] = softmax(draft row / T_r)[d] for k < n_r, where the
 * row is draft_row0[r] + k of draft_logits (row_stride elements per row),
 * d = draft_tokens[r * D_max + k], n_r = depth[r] (depth NULL: D_max) and
 * T_r = temperature[r], read as 1 when it is 0 (a greedy drafter is scored
 * by its softmax probability).  conf is 0 for k >= n_r and NaN where the row
 * has a NaN or +inf or is all -inf, d is outside [0, V), or the request's
 * temperature or depth is invalid (sv_allocate_budget reads NaN as 0).
 *
 * All arrays are device memory owned by the caller; conf is float [B, D_max].
 * Layout requirements as for sv_verify_batch (16-byte aligned logits,
 * row_stride a multiple of 8 (bf16) / 4 (fp32) elements, >= V).  workspace:
 * device memory of at least sv_draft_confidence_workspace_bytes bytes,
 * 256-byte aligned, scratch.  Errors: SV_ERR_INVALID_ARGUMENT for bad sizes
 * or null pointers, SV_ERR_UNSUPPORTED for the dtype or layout,
 * SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_DEVICE if a launch fails; nothing is
 * launched on an error.  Stream-ordered, no host synchronisation.
 * ------------------------------------------------------------------------- */
size_t sv_draft_confidence_workspace_bytes(sv_dtype dtype, int32_t B, int32_t D_max, int64_t V);

sv_status sv_draft_confidence(sv_dtype dtype, int32_t B, int32_t D_max, int64_t V,
                              int64_t row_stride, const void* draft_logits,
                              const int64_t* draft_row0, const int32_t* draft_tokens,
                              const int32_t* depth, const float* temperature, float* conf,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sv_select_budget_ratio -- D-cut's keep ratio ("AngelSpec: specialize the
 * drafter...", section "D-cut": each step the ratio is chosen among a few
 * values, by default 0.25, 0.5, 0.75 and 1, from a runtime latency table
 * profiled across batch sizes and keep ratios, as the one that maximises
 * projected throughput; Figure 3 panel 2), followed by the budget of
 * sv_allocate_budget at the chosen K.
 *
 * With N = sum over requests of min(max(max_depth[r], 0), D_max) drafted
 * positions, ratio j keeps K_j = ceil(ratios[j] * N) positions and projects
 * (B + U_j) / latency_j tokens per unit time, U_j the kept utility (the sum
 * of the kept prefix-confidence products).  latency_j comes from the host
 * table table_latency[i * n_ratios + j] (n_batch rows, table_batch[i]
 * strictly ascending batch sizes), linearly interpolated in B between the
 * two nearest sizes and clamped at the ends.  The first j with the largest
 * projected value is chosen.
 *
 * Host inputs: ratios [n_ratios] in [0, 1], 1 <= n_ratios <= SV_MAX_RATIOS;
 * table_batch [n_batch]; table_latency [n_batch * n_ratios], finite and > 0.
 * Device inputs: conf [B, D_max], max_depth [B] or NULL.  Device outputs:
 * choice [1], K_chosen [1], projected [n_ratios] (optional), and depth,
 * draft_row0, target_row0, utility as sv_allocate_budget.  Requires
 * B * D_max <= SV_MAX_BUDGET_POSITIONS.  Errors: SV_ERR_INVALID_ARGUMENT
 * before any launch, SV_ERR_DEVICE if the launch fails.
 * ------------------------------------------------------------------------- */
#define SV_MAX_RATIOS 8

sv_status sv_select_budget_ratio(const float* conf, int32_t B, int32_t D_max,
                                 const int32_t* max_depth, int32_t n_ratios,
                                 const double* ratios, int32_t n_batch,
                                 const int32_t* table_batch, const float* table_latency,
                                 int32_t* choice, int64_t* K_chosen, float* projected,
                                 int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                                 float* utility, void* stream);

/* ---------------------------------------------------------------------------
 * sv_sample_rows -- one token per request drawn from softmax(row / T) on the
 * verifier's Philox stream: the drafter's step of the decode loop ("AngelSpec:
 * specialize the drafter...", section "MTP": the drafter proposes a block that
 * the target verifies in one pass; tradepoint.io page, "The MTP path":
 * acceptance measured over whole generations).
 *
 * Request r draws from row row_base + row_index[r * index_stride] of logits
 * (row_stride elements per row; the caller guarantees the row exists) with
 * u = (w2 >> 8) * 2^-24, w2 word 2 of Philox4x32-10(key = (seed low, seed
 * high), counter = (position, request_id[r], step, 0)) -- words 0 and 1 of
 * that block are sv_verify_batch's accept and draw uniforms at the same
 * position.  The token is the smallest y whose cumulative weight exceeds
 * u * R, weights exp((x - max) / T) in float64 and R their sum; at T = 0 the
 * first arg max.  tokens[r * token_stride] receives it, or -1 when
 * row_index is negative, the temperature is negative, NaN or infinite, or
 * the row holds a NaN or +inf or only -inf.  Strides let successive calls
 * chain a drafter: call k reads the tokens call k - 1 wrote.
 *
 * Device arrays owned by the caller: row_index, temperature, request_id
 * (NULL: r), tokens.  Errors: SV_ERR_UNSUPPORTED (dtype),
 * SV_ERR_INVALID_ARGUMENT (sizes, strides, null pointers) before any launch;
 * SV_ERR_DEVICE if the launch fails.  One workgroup per request.
 * ------------------------------------------------------------------------- */
sv_status sv_sample_rows(sv_dtype dtype, int32_t B, int64_t V, int64_t row_stride,
                         const void* logits, int64_t row_base, const int32_t* row_index,
                         int64_t index_stride, const float* temperature,
                         const uint32_t* request_id, uint64_t seed, uint32_t step,
                         uint32_t position, int32_t* tokens, int64_t token_stride, void* stream);

/* ---------------------------------------------------------------------------
 * sv_stream_read -- calibration, not part of the method: reads `bytes` bytes
 * of device memory at `buf` once (16-byte vector loads, grid-stride over
 * blocks_per_cu 256-thread workgroups per compute unit) and folds them by xor
 * into sink[0] (one atomic per workgroup; sink is device memory of one
 * uint32).  Its time gives the HBM read rate this chip reaches with no
 * arithmetic and no writes, the practical ceiling of the row passes, which
 * read each logit row once.  buf 16-byte aligned, bytes a multiple of 16,
 * 1 <= blocks_per_cu <= 32; else SV_ERR_INVALID_ARGUMENT before any launch.
 * ------------------------------------------------------------------------- */
sv_status sv_stream_read(const void* buf, size_t bytes, int32_t blocks_per_cu, uint32_t* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
