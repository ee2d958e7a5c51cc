/*
 * svo.c -- CPU oracle for batched lossless draft verification and the
 * batch-shared verification budget.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Plain C, single
 * threaded, built without fast-math and without FMA contraction.
 *
 * Every function states the passage of the AngelSpec pages it follows; the
 * pages are named in svo.h.
 */
#include "svo.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Philox4x32-10.  Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11, section on the Philox family: each round multiplies
 * counter words 0 and 2 by two fixed 32-bit multipliers, keeps the 64-bit
 * products' high and low halves, and forms the next counter from the high
 * halves xored with the other two counter words and the round key, plus the
 * low halves; the key is bumped by two Weyl constants (golden ratio and
 * sqrt(3) - 1 in 0.32 fixed point) between rounds. */

static const uint32_t PHILOX_MUL_A = 0xD2511F53u;
static const uint32_t PHILOX_MUL_B = 0xCD9E8D57u;
static const uint32_t PHILOX_WEYL_A = 0x9E3779B9u;
static const uint32_t PHILOX_WEYL_B = 0xBB67AE85u;

void svo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_WEYL_A;
      k1 += PHILOX_WEYL_B;
    }
    uint64_t prod_a = (uint64_t)PHILOX_MUL_A * (uint64_t)c0;
    uint64_t prod_b = (uint64_t)PHILOX_MUL_B * (uint64_t)c2;
    uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
    uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
    uint32_t n0 = hi_b ^ c1 ^ k0;
    uint32_t n1 = lo_b;
    uint32_t n2 = hi_a ^ c3 ^ k1;
    uint32_t n3 = lo_a;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

double svo_u24(uint32_t w) { return (double)(w >> 8) * (1.0 / 16777216.0); }

void svo_uniforms(uint64_t seed, uint32_t request_id, uint32_t step, uint32_t position,
                  double* u_accept, double* u_sample) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {position, request_id, step, 0u};
  uint32_t w[4];
  svo_philox4x32_10(ctr, key, w);
  if (u_accept) *u_accept = svo_u24(w[0]);
  if (u_sample) *u_sample = svo_u24(w[1]);
}

/* ------------------------------------------------------------------------- */
/* One row.  p = softmax(x / T) over the whole vocabulary (tradepoint.io page,
 * "Why one universal drafter underperforms": the target scores every drafted
 * position in one pass). */

int svo_row_valid(const float* x, int64_t V) {
  int finite_seen = 0;
  for (int64_t y = 0; y < V; ++y) {
    float v = x[y];
    if (isnan(v)) return 0;
    if (isinf(v)) {
      if (v > 0) return 0;
      continue;
    }
    finite_seen = 1;
  }
  return finite_seen;
}

/* |m * sl| < 2^24 in float32 for the row maximum m (a valid row). */
static int svo_scale_ok(const float* x, int64_t V, float sl) {
  float m = -INFINITY;
  for (int64_t y = 0; y < V; ++y)
    if (x[y] > m) m = x[y];
  const float scaled = m * sl;
  return fabsf(scaled) < 16777216.0f;
}

int64_t svo_argmax(const float* x, int64_t V) {
  int64_t best = -1;
  for (int64_t y = 0; y < V; ++y) {
    if (isnan(x[y])) continue;
    if (best < 0 || x[y] > x[best]) best = y;
  }
  return best;
}

static double row_max(const float* x, int64_t V) {
  double m = -INFINITY;
  for (int64_t y = 0; y < V; ++y)
    if ((double)x[y] > m) m = (double)x[y];
  return m;
}

double svo_log_normalizer(const float* x, int64_t V, double T) {
  double m = row_max(x, V);
  long double z = 0.0L;
  for (int64_t y = 0; y < V; ++y) z += expl(((long double)x[y] - (long double)m) / (long double)T);
  return (double)((long double)m / (long double)T + logl(z));
}

/* log softmax(x / T)[y] given the log normaliser. */
static long double log_prob(const float* x, double lognorm, double T, int64_t y) {
  return (long double)x[y] / (long double)T - (long double)lognorm;
}

double svo_prob(const float* x, int64_t V, double T, int64_t y) {
  double L = svo_log_normalizer(x, V, T);
  return (double)expl(log_prob(x, L, T, y));
}

/* "AngelSpec: specialize the drafter..." section "MTP: fix position 2 and 3":
 * the per-position acceptance rate alpha in equation L_e2e, read as the
 * probability that the accept test passes, sum_y q(y) min(1, p(y)/q(y)) =
 * sum_y min(p(y), q(y)) = 1 - TV(p, q) (the page ties the objective to total
 * variation). */
double svo_alpha(const float* P, const float* Q, int64_t V, double T) {
  double LP = svo_log_normalizer(P, V, T);
  double LQ = svo_log_normalizer(Q, V, T);
  long double a = 0.0L;
  for (int64_t y = 0; y < V; ++y) {
    long double p = expl(log_prob(P, LP, T, y));
    long double q = expl(log_prob(Q, LQ, T, y));
    a += (p < q) ? p : q;
  }
  return (double)a;
}

/* Accept test of the standard rejection-sampling rule (tradepoint.io page,
 * "Why one universal drafter underperforms"): keep draft token d when
 * u < min(1, p(d) / q(d)); with u < 1 the min is implied. */
int svo_accept(const float* P, const float* Q, int64_t V, double T, int32_t d, double u,
               double* ratio) {
  double LP = svo_log_normalizer(P, V, T);
  double LQ = svo_log_normalizer(Q, V, T);
  long double lp = log_prob(P, LP, T, d);
  long double lq = log_prob(Q, LQ, T, d);
  long double r;
  if (isinf((double)lp) && lp < 0) r = 0.0L;          /* p(d) = 0: never kept   */
  else if (isinf((double)lq) && lq < 0) r = INFINITY; /* q(d) = 0 < p(d): kept  */
  else r = expl(lp - lq);
  if (ratio) *ratio = (double)r;
  return (long double)u < r;
}

/* Inverse CDF over non-negative weights w[0..V-1] with total R: the smallest y
 * whose running sum exceeds t = u * R; if rounding leaves t at or above the
 * total, the last token of non-zero weight. */
static int64_t inverse_cdf(const long double* w, int64_t V, long double R, double u,
                           double* margin) {
  long double t = (long double)u * R;
  long double c = 0.0L;
  int64_t last_nonzero = -1;
  for (int64_t y = 0; y < V; ++y) {
    long double before = c;
    c += w[y];
    if (w[y] > 0.0L) last_nonzero = y;
    if (c > t) {
      long double lo = t - before, hi = c - t;
      if (margin) *margin = (double)(lo < hi ? lo : hi);
      return y;
    }
  }
  if (margin) *margin = 0.0;
  return last_nonzero;
}

/* Correction draw after a rejection: normalize(max(0, p - q)) (the standard
 * rule behind "rejection sampling ... lossless", tradepoint.io page). */
int64_t svo_sample_residual(const float* P, const float* Q, int64_t V, double T, double u,
                            double* margin, double* residual_mass) {
  double LP = svo_log_normalizer(P, V, T);
  double LQ = svo_log_normalizer(Q, V, T);
  long double* w = (long double*)malloc(sizeof(long double) * (size_t)V);
  long double R = 0.0L;
  for (int64_t y = 0; y < V; ++y) {
    long double p = expl(log_prob(P, LP, T, y));
    long double q = expl(log_prob(Q, LQ, T, y));
    w[y] = (p > q) ? (p - q) : 0.0L;
    R += w[y];
  }
  if (residual_mass) *residual_mass = (double)R;
  int64_t y;
  if (R > 0.0L) {
    y = inverse_cdf(w, V, R, u, margin);
  } else {
    /* R = 0 means p = q everywhere; a rejection cannot happen in exact
     * arithmetic, so the draw falls back to p. */
    R = 0.0L;
    for (int64_t i = 0; i < V; ++i) {
      w[i] = expl(log_prob(P, LP, T, i));
      R += w[i];
    }
    y = inverse_cdf(w, V, R, u, margin);
  }
  free(w);
  return y;
}

/* Bonus draw after a fully accepted block: one token from p. */
int64_t svo_sample_target(const float* P, int64_t V, double T, double u, double* margin) {
  double LP = svo_log_normalizer(P, V, T);
  long double* w = (long double*)malloc(sizeof(long double) * (size_t)V);
  long double R = 0.0L;
  for (int64_t y = 0; y < V; ++y) {
    w[y] = expl(log_prob(P, LP, T, y));
    R += w[y];
  }
  int64_t yv = inverse_cdf(w, V, R, u, margin);
  free(w);
  return yv;
}

/* Equation L_e2e ("MTP: fix position 2 and 3"): the inner sum
 * sum_{m=0}^{D-1} prod_{k=0}^{m} alpha_k is the expected accepted length,
 * a product because one rejection invalidates every later position. */
double svo_expected_accepted(const double* alpha, int32_t n) {
  double total = 0.0, prefix = 1.0;
  for (int32_t m = 0; m < n; ++m) {
    prefix *= alpha[m];
    total += prefix;
  }
  return total;
}

/* ------------------------------------------------------------------------- */
/* One request (tradepoint.io page, "Why one universal drafter
 * underperforms": the target verifies the drafted tokens together with
 * rejection sampling; "AngelSpec: specialize the drafter..." section "MTP":
 * one rejection invalidates every position after it).  Positions are tested
 * in order; the first rejection ends the block and its position emits a
 * correction token; a block with no rejection emits a bonus token from the
 * row after the last draft.  At T = 0 ("The MTP path": results at T = 0, the
 * drafter feeds its arg max forward) the test is an arg-max match and the
 * emitted token at the stop position is the target's arg max. */
int32_t svo_verify_request(const float* const* P_rows, const float* const* Q_rows,
                           const int32_t* d, int32_t n, int64_t V, float T,
                           const double* u_accept, const double* u_sample, int32_t* out,
                           double* accept_margin, double* draw_margin, uint32_t* bits) {
  double amargin = INFINITY, dmargin = INFINITY;
  int32_t tau = n;
  if (T == 0.0f) {
    for (int32_t k = 0; k < n; ++k) {
      if ((int64_t)d[k] != svo_argmax(P_rows[k], V)) {
        tau = k;
        break;
      }
    }
    for (int32_t k = 0; k < tau; ++k) out[k] = d[k];
    out[tau] = (int32_t)svo_argmax(P_rows[tau], V);
  } else {
    double Td = (double)T;
    int64_t y = -1;
    for (int32_t k = 0; k < n; ++k) {
      double ratio;
      int keep = svo_accept(P_rows[k], Q_rows[k], V, Td, d[k], u_accept[k], &ratio);
      double gap = fabs(u_accept[k] - ratio);
      if (gap < amargin) amargin = gap;
      if (!keep) {
        double mass;
        tau = k;
        y = svo_sample_residual(P_rows[k], Q_rows[k], V, Td, u_sample[k], &dmargin, &mass);
        if (mass <= 0.0 && bits) *bits |= SVO_BIT_RESIDUAL_ZERO;
        break;
      }
    }
    if (tau == n) y = svo_sample_target(P_rows[n], V, Td, u_sample[n], &dmargin);
    for (int32_t k = 0; k < tau; ++k) out[k] = d[k];
    out[tau] = (int32_t)y;
  }
  if (accept_margin) *accept_margin = amargin;
  if (draw_margin) *draw_margin = dmargin;
  return tau;
}

int svo_verify_batch(const float* target, const float* draft, int64_t V, int64_t row_stride,
                     const int64_t* target_row0, const int64_t* draft_row0,
                     const int32_t* draft_tokens, const int32_t* depth,
                     const float* temperature, const uint32_t* request_id, int32_t B,
                     int32_t D_max, uint64_t seed, uint32_t step, int32_t* accepted_len,
                     int32_t* out_tokens, int32_t* num_out, double* alpha,
                     double* accept_margin, double* draw_margin, uint32_t* bits,
                     int32_t* draws) {
  if (B < 0 || D_max < 0 || V <= 0 || row_stride < V || !target || !target_row0 ||
      !draft_tokens || !depth || !temperature || !accepted_len || !out_tokens || !num_out)
    return SVO_ERR_INVALID_ARGUMENT;

  const float** P_rows = (const float**)malloc(sizeof(float*) * (size_t)(D_max + 1));
  const float** Q_rows = (const float**)malloc(sizeof(float*) * (size_t)(D_max + 1));
  double* ua = (double*)malloc(sizeof(double) * (size_t)(D_max + 1));
  double* us = (double*)malloc(sizeof(double) * (size_t)(D_max + 1));

  for (int32_t r = 0; r < B; ++r) {
    int32_t n = depth[r];
    float T = temperature[r];
    uint32_t rid = request_id ? request_id[r] : (uint32_t)r;
    const int32_t* d = draft_tokens + (int64_t)r * D_max;
    int32_t* out = out_tokens + (int64_t)r * (D_max + 1);
    uint32_t b = 0;
    for (int32_t k = 0; k <= D_max; ++k) out[k] = -1;
    if (alpha)
      for (int32_t k = 0; k < D_max; ++k) alpha[(int64_t)r * D_max + k] = 0.0;
    accepted_len[r] = 0;
    num_out[r] = 0;
    if (accept_margin) accept_margin[r] = INFINITY;
    if (draw_margin) draw_margin[r] = INFINITY;
    if (draws) draws[r] = 0;

    if (n < 0 || n > D_max) b |= SVO_BIT_BAD_DEPTH;
    if (!(T >= 0.0f) || isinf(T)) b |= SVO_BIT_BAD_TEMPERATURE;
    if (!b) {
      for (int32_t k = 0; k < n; ++k)
        if (d[k] < 0 || (int64_t)d[k] >= V) b |= SVO_BIT_BAD_TOKEN;
      for (int32_t k = 0; k <= n; ++k) {
        P_rows[k] = target + (target_row0[r] + k) * row_stride;
        if (!svo_row_valid(P_rows[k], V)) b |= SVO_BIT_BAD_ROW;
      }
      if (T != 0.0f && n > 0 && !draft) {
        /* a sampling request with drafted positions needs draft rows: without
           any (allowed only for greedy batches) it is an invalid request */
        b |= SVO_BIT_BAD_ROW;
      } else if (T != 0.0f) {
        for (int32_t k = 0; k < n; ++k) {
          Q_rows[k] = draft + (draft_row0[r] + k) * row_stride;
          if (!svo_row_valid(Q_rows[k], V)) b |= SVO_BIT_BAD_ROW;
        }
      }
      if (T > 0.0f) {
        /* Domain of the temperature (a reading; the pages fix none): the
           verifier scales logits by log2(e)/T in float32 and is exact only
           while every verified row's maximum m has |m * fl(log2(e)/T)| below
           2^24, both products rounded to float32.  Past that the request is
           reported invalid; greedy verification (T = 0) covers that regime. */
        const float sl = 1.4426950408889634f / T;
        for (int32_t k = 0; k <= n; ++k)
          if (svo_row_valid(P_rows[k], V) && !svo_scale_ok(P_rows[k], V, sl))
            b |= SVO_BIT_BAD_TEMPERATURE;
        if (draft)
          for (int32_t k = 0; k < n; ++k)
            if (svo_row_valid(Q_rows[k], V) && !svo_scale_ok(Q_rows[k], V, sl))
              b |= SVO_BIT_BAD_TEMPERATURE;
      }
    }
    if (b) {
      if (bits) bits[r] = b;
      continue;
    }

    for (int32_t k = 0; k <= n; ++k) svo_uniforms(seed, rid, step, (uint32_t)k, &ua[k], &us[k]);
    double am, dm;
    int32_t tau =
        svo_verify_request(P_rows, Q_rows, d, n, V, T, ua, us, out, &am, &dm, &b);
    accepted_len[r] = tau;
    num_out[r] = tau + 1;
    if (accept_margin) accept_margin[r] = am;
    if (draw_margin) draw_margin[r] = dm;
    if (draws) draws[r] = (T == 0.0f) ? 0 : ((tau < n ? tau + 1 : n) + 1);
    if (bits) bits[r] = b;
    if (alpha) {
      for (int32_t k = 0; k < n; ++k) {
        double a;
        if (T == 0.0f)
          /* Greedy drafting: q is the point mass at d, p the point mass at
           * the target arg max, so sum min(p, q) is 1 on a match, else 0. */
          a = ((int64_t)d[k] == svo_argmax(P_rows[k], V)) ? 1.0 : 0.0;
        else
          a = svo_alpha(P_rows[k], Q_rows[k], V, (double)T);
        alpha[(int64_t)r * D_max + k] = a;
      }
    }
  }
  free(P_rows);
  free(Q_rows);
  free(ua);
  free(us);
  return SVO_OK;
}

/* ------------------------------------------------------------------------- */
/* Verification budget ("AngelSpec: specialize the drafter..." section
 * "D-cut": equation K_rho). */
int64_t svo_k_rho(int32_t B, int32_t D, double rho) {
  double k = ceil(rho * (double)B * (double)(D + 1));
  int64_t kk = (int64_t)k;
  return kk > B ? kk : (int64_t)B;
}

typedef struct {
  float s;
  int32_t r, k;
} scored_pos;

/* Order of Figure 3 panel 3 ("flattened, sorted by confidence"): higher score
 * first; equal scores by lower request, then lower position. */
static int by_score_desc(const void* a, const void* b) {
  const scored_pos* x = (const scored_pos*)a;
  const scored_pos* y = (const scored_pos*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  if (x->r != y->r) return x->r < y->r ? -1 : 1;
  if (x->k != y->k) return x->k < y->k ? -1 : 1;
  return 0;
}

/* Section "D-cut": equation A-hat sums the prefix-confidence products
 * s_{i,k} of the kept positions; Figure 3 flattens every (request, position)
 * of the batch, sorts by that score and keeps a global top-K, so each
 * request's kept depth is however many of its positions survive. */
int svo_allocate_budget(const float* conf, int32_t B, int32_t D_max, const int32_t* max_depth,
                        int64_t K, int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                        double* utility) {
  if (B < 0 || D_max < 0 || !depth || (B > 0 && D_max > 0 && !conf))
    return SVO_ERR_INVALID_ARGUMENT;
  scored_pos* all = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(B * D_max + 1));
  int64_t count = 0;
  double total = 0.0;
  for (int32_t r = 0; r < B; ++r) {
    int32_t lim = max_depth ? max_depth[r] : D_max;
    if (lim < 0) lim = 0;
    if (lim > D_max) lim = D_max;
    float s = 1.0f;
    for (int32_t k = 0; k < lim; ++k) {
      float c = conf[(int64_t)r * D_max + k];
      if (!(c >= 0.0f)) c = 0.0f; /* NaN and negatives read as 0 */
      if (c > 1.0f) c = 1.0f;
      s = s * c;
      all[count].s = s;
      all[count].r = r;
      all[count].k = k;
      ++count;
      total += (double)s;
    }
  }
  if (K < 0) K = 0;
  if (K > count) K = count;
  qsort(all, (size_t)count, sizeof(scored_pos), by_score_desc);
  for (int32_t r = 0; r < B; ++r) depth[r] = 0;
  double kept = 0.0;
  for (int64_t i = 0; i < K; ++i) {
    depth[all[i].r] += 1;
    kept += (double)all[i].s;
  }
  int64_t dr = 0, tr = 0;
  for (int32_t r = 0; r < B; ++r) {
    if (draft_row0) draft_row0[r] = dr;
    if (target_row0) target_row0[r] = tr;
    dr += depth[r];
    tr += depth[r] + 1;
  }
  if (utility) {
    utility[0] = kept;
    utility[1] = total;
  }
  free(all);
  return SVO_OK;
}

/* Section "D-cut", the budget widget: the fixed allocation cuts every request
 * at the same position for the same total K. */
void svo_fixed_depth(int32_t B, int32_t D_max, int64_t K, int32_t* depth) {
  if (B <= 0) return;
  int64_t base = K / B, extra = K % B;
  for (int32_t r = 0; r < B; ++r) {
    int64_t n = base + (r < extra ? 1 : 0);
    if (n > D_max) n = D_max;
    if (n < 0) n = 0;
    depth[r] = (int32_t)n;
  }
}

/* The fixed-depth baseline's allocation and utility: the depths of
 * svo_fixed_depth, row offsets as svo_allocate_budget writes them, and
 * utility = (sum of the prefix-confidence products of the kept positions,
 * sum over every position), the products taken as in svo_allocate_budget.
 * The budget widget of section "D-cut" compares the first with the global
 * top-K's at the same K (utility retained, global vs fixed). */
int svo_fixed_depth_budget(const float* conf, int32_t B, int32_t D_max, int64_t K, int32_t* depth,
                           int64_t* draft_row0, int64_t* target_row0, double* utility) {
  if (B < 0 || D_max < 0 || !depth || (B > 0 && D_max > 0 && !conf))
    return SVO_ERR_INVALID_ARGUMENT;
  svo_fixed_depth(B, D_max, K, depth);
  double kept = 0.0, total = 0.0;
  int64_t dr = 0, tr = 0;
  for (int32_t r = 0; r < B; ++r) {
    float s = 1.0f;
    for (int32_t k = 0; k < D_max; ++k) {
      float c = conf[(int64_t)r * D_max + k];
      if (!(c >= 0.0f)) c = 0.0f; /* NaN and negatives read as 0 */
      if (c > 1.0f) c = 1.0f;
      s = s * c;
      total += (double)s;
      if (k < depth[r]) kept += (double)s;
    }
    if (draft_row0) draft_row0[r] = dr;
    if (target_row0) target_row0[r] = tr;
    dr += depth[r];
    tr += depth[r] + 1;
  }
  if (utility) {
    utility[0] = kept;
    utility[1] = total;
  }
  return SVO_OK;
}

/* ------------------------------------------------------------------------- */
/* Statistics: equation L_e2e (expected accepted length) and the MAL /
 * mean-acceptance figures of "The MTP path" (tradepoint.io page), whose
 * printed values satisfy MAL = 1 + D * mean acceptance.  A request has at
 * most D_max draft positions, so a depth outside [0, D_max] counts as the
 * nearest end of that range. */
static int32_t svo_clamp_depth(int32_t n, int32_t D_max) {
  return n < 0 ? 0 : (n > D_max ? D_max : n);
}

int svo_accept_stats(const int32_t* depth, const double* alpha, const int32_t* accepted_len,
                     int32_t B, int32_t D_max, double* expected_len, double* per_depth,
                     double* summary) {
  if (B < 0 || D_max < 0 || !depth || !accepted_len) return SVO_ERR_INVALID_ARGUMENT;
  if (per_depth)
    for (int32_t i = 0; i < 3 * D_max; ++i) per_depth[i] = 0.0;
  double sum_tau = 0.0, sum_n = 0.0, sum_e = 0.0;
  for (int32_t r = 0; r < B; ++r) {
    int32_t n = svo_clamp_depth(depth[r], D_max), tau = accepted_len[r];
    double e = alpha ? svo_expected_accepted(alpha + (int64_t)r * D_max, n) : 0.0;
    if (expected_len) expected_len[r] = e;
    sum_e += e;
    sum_tau += tau;
    sum_n += n;
    if (per_depth) {
      for (int32_t k = 0; k < n; ++k) {
        if (tau >= k) per_depth[k] += 1.0;
        if (tau > k) per_depth[D_max + k] += 1.0;
        if (alpha) per_depth[2 * D_max + k] += alpha[(int64_t)r * D_max + k];
      }
    }
  }
  if (per_depth) {
    for (int32_t k = 0; k < D_max; ++k) {
      int32_t with_k = 0;
      for (int32_t r = 0; r < B; ++r)
        if (svo_clamp_depth(depth[r], D_max) > k) ++with_k;
      per_depth[2 * D_max + k] = with_k ? per_depth[2 * D_max + k] / with_k : 0.0;
    }
  }
  if (summary) {
    summary[0] = B ? 1.0 + sum_tau / B : 0.0;
    summary[1] = B ? 1.0 + sum_e / B : 0.0;
    summary[2] = sum_n > 0 ? sum_tau / sum_n : 0.0;
    summary[3] = sum_n;
  }
  return SVO_OK;
}

/* Statistics over many verified batches (the decode loop's steps), as the
 * tradepoint.io page, "The MTP path", reports them over whole generations:
 * MAL, mean acceptance and position-wise acceptance.  accum (length
 * 3 + 2 D_max) is added to: accum[0] += sum of (tau + 1) (tokens emitted),
 * accum[1] += B, accum[2] += sum of E[tau_r] (0 without alpha),
 * accum[3 + k] += #requests with depth > k (position k verified),
 * accum[3 + D_max + k] += #requests with tau > k (position k accepted), with
 * depth clamped to [0, D_max].  summary (length 3 + D_max) is then taken from
 * the totals: MAL = accum[0] / accum[1]; expected MAL = 1 + accum[2] /
 * accum[1]; mean acceptance = sum tau / sum depth; position-wise acceptance
 * at position k + 1 (1-based) = P(tau >= k + 1) = accum[3 + D_max + k] /
 * accum[1], so that MAL = 1 + the sum of the position-wise acceptances. */
int svo_accept_accumulate(const int32_t* depth, const double* alpha, const int32_t* accepted_len,
                          int32_t B, int32_t D_max, double* accum, double* summary) {
  if (B < 0 || D_max < 0 || !accum || (B > 0 && (!depth || !accepted_len)))
    return SVO_ERR_INVALID_ARGUMENT;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t n = svo_clamp_depth(depth[r], D_max);
    const int32_t tau = accepted_len[r];
    accum[0] += (double)(tau + 1);
    accum[1] += 1.0;
    if (alpha) accum[2] += svo_expected_accepted(alpha + (int64_t)r * D_max, n);
    for (int32_t k = 0; k < D_max; ++k) {
      if (n > k) accum[3 + k] += 1.0;
      if (tau > k) accum[3 + D_max + k] += 1.0;
    }
  }
  if (summary) {
    double sum_n = 0.0;
    for (int32_t k = 0; k < D_max; ++k) sum_n += accum[3 + k];
    const double req = accum[1];
    summary[0] = req > 0 ? accum[0] / req : 0.0;
    summary[1] = req > 0 ? 1.0 + accum[2] / req : 0.0;
    summary[2] = sum_n > 0 ? (accum[0] - req) / sum_n : 0.0;
    for (int32_t k = 0; k < D_max; ++k) summary[3 + k] = req > 0 ? accum[3 + D_max + k] / req : 0.0;
  }
  return SVO_OK;
}

/* ------------------------------------------------------------------------- */
/* Drafter confidence ("AngelSpec: specialize the drafter..." section "D-cut",
 * Figure 3 panel 1: the drafter emits confidence-scored candidate tokens;
 * equation A-hat multiplies these confidences along a request).  Reading:
 * the confidence of draft token d at position k is the drafter's own
 * probability of it, q_k(d) = softmax(draft row k / T)[d]; a greedy drafter
 * (T = 0) is scored by its softmax at T = 1.  NaN marks an invalid row,
 * token, depth or temperature (the budget reads NaN as 0); positions at or
 * past the request's depth get 0. */
int svo_draft_confidence(const float* draft, int64_t V, int64_t row_stride, int32_t B,
                         int32_t D_max, const int64_t* draft_row0, const int32_t* draft_tokens,
                         const int32_t* depth, const float* temperature, float* conf) {
  if (B < 0 || D_max < 0 || V < 1 || row_stride < V || !conf) return SVO_ERR_INVALID_ARGUMENT;
  if (B > 0 && D_max > 0 && (!draft || !draft_row0 || !draft_tokens || !temperature))
    return SVO_ERR_INVALID_ARGUMENT;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t n = depth ? depth[r] : D_max;
    const double T = (double)temperature[r];
    const int bad_request = n < 0 || n > D_max || !(T >= 0.0) || isinf(T);
    const double Te = T > 0.0 ? T : 1.0;
    for (int32_t k = 0; k < D_max; ++k) {
      float* out = &conf[(int64_t)r * D_max + k];
      if (bad_request) {
        *out = NAN;
        continue;
      }
      if (k >= n) {
        *out = 0.0f;
        continue;
      }
      const float* row = draft + (draft_row0[r] + k) * row_stride;
      const int32_t d = draft_tokens[(int64_t)r * D_max + k];
      if (d < 0 || (int64_t)d >= V || !svo_row_valid(row, V)) {
        *out = NAN;
        continue;
      }
      *out = (float)svo_prob(row, V, Te, d);
    }
  }
  return SVO_OK;
}

/* ------------------------------------------------------------------------- */
/* D-cut's keep ratio ("AngelSpec: specialize the drafter..." section
 * "D-cut": each step the ratio is chosen among a few values, by default
 * 0.25, 0.5, 0.75 and 1, from a runtime cost table profiled across batch
 * sizes and keep ratios (Figure 3 panel 2), as the one that maximises
 * projected throughput rather than kept length).  Readings:
 *  - ratio j keeps K_j = ceil(rho_j * N) draft positions, N = the number of
 *    drafted positions (sum of the depth limits), since K counts draft
 *    positions (the budget widget keeps 24 of 48 at rho = 1/2);
 *  - projected tokens of ratio j = B + U_j, U_j = the kept utility of the
 *    global top-K_j (equation A-hat summed over the batch: expected accepted
 *    drafts) plus the one token every request emits;
 *  - its latency is the table's, linearly interpolated in the batch size
 *    between the two nearest profiled sizes and clamped at the ends;
 *  - the first ratio (in the given order) with the largest tokens / latency
 *    wins, and its allocation is returned. */
double svo_table_latency(int32_t n_batch, const int32_t* table_batch, const float* table_latency,
                         int32_t n_ratios, int32_t j, int32_t B) {
  if (B <= table_batch[0]) return (double)table_latency[j];
  if (B >= table_batch[n_batch - 1]) return (double)table_latency[(int64_t)(n_batch - 1) * n_ratios + j];
  int32_t i = 0;
  while (table_batch[i + 1] < B) ++i;
  const double lo = (double)table_latency[(int64_t)i * n_ratios + j];
  const double hi = (double)table_latency[(int64_t)(i + 1) * n_ratios + j];
  const double f = (double)(B - table_batch[i]) / (double)(table_batch[i + 1] - table_batch[i]);
  return lo + (hi - lo) * f;
}

int svo_select_budget_ratio(const float* conf, int32_t B, int32_t D_max, const int32_t* max_depth,
                            int32_t n_ratios, const double* ratios, int32_t n_batch,
                            const int32_t* table_batch, const float* table_latency,
                            int32_t* choice, int64_t* K_chosen, double* projected,
                            int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                            double* utility) {
  if (B < 0 || D_max < 0 || n_ratios < 1 || n_batch < 1 || !ratios || !table_batch ||
      !table_latency || !choice || !K_chosen || !depth)
    return SVO_ERR_INVALID_ARGUMENT;
  for (int32_t j = 0; j < n_ratios; ++j)
    if (!(ratios[j] >= 0.0 && ratios[j] <= 1.0)) return SVO_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < n_batch; ++i) {
    if (i > 0 && !(table_batch[i] > table_batch[i - 1])) return SVO_ERR_INVALID_ARGUMENT;
    for (int32_t j = 0; j < n_ratios; ++j) {
      const float l = table_latency[(int64_t)i * n_ratios + j];
      if (!(l > 0.0f) || isinf(l)) return SVO_ERR_INVALID_ARGUMENT;
    }
  }
  int64_t N = 0;
  for (int32_t r = 0; r < B; ++r) {
    int32_t lim = max_depth ? max_depth[r] : D_max;
    if (lim < 0) lim = 0;
    if (lim > D_max) lim = D_max;
    N += lim;
  }
  int32_t best = -1;
  double best_tp = 0.0;
  for (int32_t j = 0; j < n_ratios; ++j) {
    const int64_t K = (int64_t)ceil(ratios[j] * (double)N);
    double u[2];
    int st = svo_allocate_budget(conf, B, D_max, max_depth, K, depth, NULL, NULL, u);
    if (st != SVO_OK) return st;
    const double lat = svo_table_latency(n_batch, table_batch, table_latency, n_ratios, j, B);
    const double tp = ((double)B + u[0]) / lat;
    if (projected) projected[j] = tp;
    if (best < 0 || tp > best_tp) {
      best = j;
      best_tp = tp;
    }
  }
  *choice = best;
  *K_chosen = (int64_t)ceil(ratios[best] * (double)N);
  return svo_allocate_budget(conf, B, D_max, max_depth, *K_chosen, depth, draft_row0, target_row0,
                             utility);
}
