/*
 * svo.h -- CPU oracle for batched lossless draft verification and the
 * batch-shared verification budget ("D-cut").
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, plain, single-threaded
 * statement of what the GPU path must compute.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * Sources (the AngelSpec pages):
 *  - "AngelSpec: specialize the drafter, share the verification budget"
 *    (ai.thesatyajit.com), intro: the target verifies every drafted token in one
 *    pass and only ever emits what it would have sampled itself; section
 *    "MTP: fix position 2 and 3", equation L_e2e and the sentence after it: one
 *    rejection invalidates every later position, so accepted length is a sum
 *    of prefix products of per-position acceptance rates; section "D-cut",
 *    Figure 3 and the equations for A-hat and K_rho: per-request prefix
 *    confidence products, flattened over the batch and cut by a global top-K.
 *  - "Tencent open-sources AngelSpec" (tradepoint.io), section "Why one
 *    universal drafter underperforms": verification is rejection sampling in
 *    one target forward and is lossless; section "The MTP path": the T=0
 *    (greedy, arg max) setting and the MAL / mean-acceptance figures.
 *  - "AngelSpec: Towards Real-World High Performance Inference..." (newx.sg),
 *    Abstract: the target distribution is not changed.
 * The accept rule u < min(1, p/q), the residual normalize(max(0, p - q)), the
 * bonus draw from p and the Philox stream are the standard speculative
 * sampling rule that the pages call lossless rejection sampling; the pages do
 * not print them.
 *
 * Arithmetic: logits arrive as IEEE float32 (bfloat16 logits are widened
 * exactly).  Per-element values are double, every sum is long double (x87
 * 80-bit), the temperature is applied as an exact division by the float32
 * temperature value.  The budget's prefix products are float32, because they
 * decide an integer selection and the GPU takes that decision in float32.
 */
#ifndef SVO_H
#define SVO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (host-side argument errors only). */
enum { SVO_OK = 0, SVO_ERR_INVALID_ARGUMENT = 1 };

/* Per-request diagnostic bits. */
enum {
  SVO_BIT_BAD_DEPTH = 1u,      /* depth outside [0, D_max]                       */
  SVO_BIT_BAD_TOKEN = 2u,      /* a draft token id outside [0, V)                */
  SVO_BIT_BAD_ROW = 4u,        /* a verified row holds NaN / +inf, or only -inf  */
  SVO_BIT_RESIDUAL_ZERO = 8u,  /* residual mass was zero; the target row was used */
  SVO_BIT_BAD_TEMPERATURE = 16u /* temperature negative, NaN or infinite, or so
                                   small that a verified row's maximum m gives
                                   |m * fl(log2(e)/T)| >= 2^24 in float32       */
};

/* ---- counter-based random numbers ---------------------------------------- */

/* Philox4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11). */
void svo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* u = (w >> 8) * 2^-24: a uniform on the 2^-24 grid in [0, 1 - 2^-24]. */
double svo_u24(uint32_t w);

/* The two uniforms of one (request, position): key = (seed low word, seed high
 * word), counter = (position, request_id, step, 0).  Word 0 feeds the accept
 * test at that position; word 1 feeds the correction / bonus draw when the
 * emitted token is drawn at that position. */
void svo_uniforms(uint64_t seed, uint32_t request_id, uint32_t step, uint32_t position,
                  double* u_accept, double* u_sample);

/* ---- one row -------------------------------------------------------------- */

/* 1 if every element is finite or -inf and at least one is finite, else 0. */
int svo_row_valid(const float* x, int64_t V);

/* Smallest index of the largest element (NaN never wins). */
int64_t svo_argmax(const float* x, int64_t V);

/* ln sum_y exp(x_y / T) for T > 0 (log normaliser of softmax(x / T)). */
double svo_log_normalizer(const float* x, int64_t V, double T);

/* softmax(x / T)[y]. */
double svo_prob(const float* x, int64_t V, double T, int64_t y);

/* Acceptance rate sum_y min(p(y), q(y)), p = softmax(P/T), q = softmax(Q/T). */
double svo_alpha(const float* P, const float* Q, int64_t V, double T);

/* Accept test for draft token d at one position: 1 if u < p(d) / q(d).
 * *ratio receives p(d)/q(d) (+inf when q(d) = 0 < p(d)). */
int svo_accept(const float* P, const float* Q, int64_t V, double T, int32_t d, double u,
               double* ratio);

/* Inverse-CDF draw from normalize(max(0, p - q)) with uniform u: the smallest y
 * whose cumulative residual mass exceeds u * R.  *margin receives the distance
 * (in probability units) from u * R to the nearest cumulative-mass boundary
 * around y; *residual_mass receives R.  If R = 0 the draw is from p. */
int64_t svo_sample_residual(const float* P, const float* Q, int64_t V, double T, double u,
                            double* margin, double* residual_mass);

/* Inverse-CDF draw from p = softmax(P/T) with uniform u (the bonus token). */
int64_t svo_sample_target(const float* P, int64_t V, double T, double u, double* margin);

/* sum_{m < n} prod_{k <= m} alpha[k]: the expected number of accepted drafts. */
double svo_expected_accepted(const double* alpha, int32_t n);

/* ---- one request with explicit uniforms ----------------------------------- */

/* Verifies one request.  P_rows[0..n] are target rows (row n is the bonus row),
 * Q_rows[0..n-1] draft rows (unused when T == 0), d[0..n-1] draft tokens.
 * u_accept[k] is the accept uniform of position k, u_sample[k] the draw
 * uniform of position k (k = 0..n).  Writes out[0..tau] (the emitted tokens)
 * and returns tau.  *draw_margin: the CDF margin of the final draw (T > 0),
 * *accept_margin: min over tested positions of |u - p/q| (T > 0). */
int32_t svo_verify_request(const float* const* P_rows, const float* const* Q_rows,
                           const int32_t* d, int32_t n, int64_t V, float T,
                           const double* u_accept, const double* u_sample, int32_t* out,
                           double* accept_margin, double* draw_margin, uint32_t* bits);

/* ---- the batch ------------------------------------------------------------- */

/* Verifies a batch (all pointers host).  Rows of request r: target rows
 * target_row0[r] + k for k = 0..depth[r], draft rows draft_row0[r] + k for
 * k < depth[r]; each row starts at row * row_stride elements.  draft_tokens is
 * [B, D_max].  Outputs: accepted_len[B], out_tokens[B, D_max + 1] (-1 padded),
 * num_out[B]; optional (may be NULL): alpha[B, D_max] (0 past depth),
 * accept_margin[B], draw_margin[B], bits[B], draws[B] (uniforms consumed). */
int svo_verify_batch(const float* target, const float* draft, int64_t V, int64_t row_stride,
                     const int64_t* target_row0, const int64_t* draft_row0,
                     const int32_t* draft_tokens, const int32_t* depth,
                     const float* temperature, const uint32_t* request_id, int32_t B,
                     int32_t D_max, uint64_t seed, uint32_t step, int32_t* accepted_len,
                     int32_t* out_tokens, int32_t* num_out, double* alpha,
                     double* accept_margin, double* draw_margin, uint32_t* bits,
                     int32_t* draws);

/* ---- the verification budget ------------------------------------------------ */

/* K_rho(B) = max(B, ceil(rho * B * (D + 1))). */
int64_t svo_k_rho(int32_t B, int32_t D, double rho);

/* Global top-K over prefix-confidence products.  conf is [B, D_max] (values
 * clamped to [0, 1], NaN read as 0); max_depth[B] (NULL = D_max) bounds each
 * request.  s[r][k] = c[r][0] * ... * c[r][k] in float32, left to right.  The
 * K (clamped to [0, sum max_depth]) largest scores are kept, ties broken by
 * lower request, then lower position.  Outputs: depth[B], draft_row0[B]
 * (exclusive scan of depth), target_row0[B] (exclusive scan of depth + 1),
 * utility[2] = (sum of kept scores, sum of all scores) (NULL allowed). */
int svo_allocate_budget(const float* conf, int32_t B, int32_t D_max, const int32_t* max_depth,
                        int64_t K, int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                        double* utility);

/* The fixed-depth baseline at the same K: every request is cut at the same
 * depth, floor(K / B), and the first K mod B requests get one more. */
void svo_fixed_depth(int32_t B, int32_t D_max, int64_t K, int32_t* depth);

/* The fixed-depth allocation at K with its row offsets (as svo_allocate_budget
 * writes them) and utility[2] = (sum of the kept positions' prefix-confidence
 * products, sum over all B * D_max positions); products as in
 * svo_allocate_budget. */
int svo_fixed_depth_budget(const float* conf, int32_t B, int32_t D_max, int64_t K, int32_t* depth,
                           int64_t* draft_row0, int64_t* target_row0, double* utility);

/* Drafter confidence: conf[r * D_max + k] = softmax(draft row / T_r)[d]
 * (T_r = 0 read as 1) for k < depth[r] (depth NULL = D_max), row
 * draft_row0[r] + k of a buffer with row_stride elements per row, d =
 * draft_tokens[r * D_max + k]; 0 for k >= depth[r]; NaN for an invalid row,
 * token, depth or temperature. */
int svo_draft_confidence(const float* draft, int64_t V, int64_t row_stride, int32_t B,
                         int32_t D_max, const int64_t* draft_row0, const int32_t* draft_tokens,
                         const int32_t* depth, const float* temperature, float* conf);

/* Latency of ratio j at batch size B from a table of n_batch ascending
 * batch sizes x n_ratios latencies (row-major): linear interpolation between
 * the two nearest sizes, clamped at the ends. */
double svo_table_latency(int32_t n_batch, const int32_t* table_batch, const float* table_latency,
                         int32_t n_ratios, int32_t j, int32_t B);

/* D-cut keep-ratio choice: for each ratio j, K_j = ceil(rho_j * N) (N = sum
 * of the depth limits), projected[j] = (B + kept utility of the top K_j) /
 * latency_j; choice = the first j with the largest projected value, K_chosen
 * = K_choice, and the allocation of svo_allocate_budget at that K. */
int svo_select_budget_ratio(const float* conf, int32_t B, int32_t D_max, const int32_t* max_depth,
                            int32_t n_ratios, const double* ratios, int32_t n_batch,
                            const int32_t* table_batch, const float* table_latency,
                            int32_t* choice, int64_t* K_chosen, double* projected,
                            int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                            double* utility);

/* ---- statistics --------------------------------------------------------------- */

/* expected_len[r] = sum_{m < n_r} prod_{k <= m} alpha[r][k];
 * per_depth[k] = #requests that tested position k, per_depth[D_max + k] =
 * #requests that accepted position k, per_depth[2 D_max + k] = mean alpha at k
 * over requests with depth > k;
 * summary = (mean(tau + 1), 1 + mean expected_len, sum tau / sum n, sum n);
 * n_r = depth[r] clamped to [0, D_max]. */
int svo_accept_stats(const int32_t* depth, const double* alpha, const int32_t* accepted_len,
                     int32_t B, int32_t D_max, double* expected_len, double* per_depth,
                     double* summary);

/* Statistics over many verified batches: adds the batch to accum
 * (3 + 2 D_max doubles: tokens emitted, requests, sum of E[tau], #verified at
 * each position, #accepted at each position) and writes, from the totals,
 * summary (3 + D_max): MAL, expected MAL, mean acceptance, and the
 * position-wise acceptance P(tau >= k) for k = 1..D_max. */
int svo_accept_accumulate(const int32_t* depth, const double* alpha, const int32_t* accepted_len,
                          int32_t B, int32_t D_max, double* accum, double* summary);

#ifdef __cplusplus
}
#endif

#endif /* SVO_H */
