// sv_budget.hip -- the batch-shared verification budget ("AngelSpec:
// specialize the drafter...", section "D-cut": Figure 3 flattens every draft
// position of the batch, sorts by confidence and keeps a global top-K;
// equation A-hat scores a request's kept prefix by its prefix-confidence
// products).
//
// One workgroup of 1024 threads: float32 prefix products, 64-bit keys
// (score bits above the complemented flat index, so equal scores order by
// lower request, then lower position), a radix select of the K-th largest
// key, per-request counts and the packed row offsets.  The whole batch
// (B * D_max <= 4096 keys, 32 KB) stays in LDS; B <= 4096.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_stats.hpp"

namespace sv {

constexpr int kBudgetThreads = 1024;
constexpr int kBudgetWaves = kBudgetThreads / kWave;
constexpr int kKeySlots = SV_MAX_BUDGET_POSITIONS / kBudgetThreads;  // keys per thread

__device__ __forceinline__ float block_sum_budget(float v, float* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < kBudgetWaves; ++w) t += lds[w];
  __syncthreads();
  return t;
}

// Inclusive prefix sum over the lanes of a wavefront.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Keys: (score bits << 32) | ~flat_index, unique and nonzero for every
// position within its request's limit, 0 elsewhere.  Within a request the
// scores do not increase with the position (confidences are clamped to
// [0, 1]) and ~index decreases, so a request's keys strictly decrease and the
// global top K keeps a prefix of every request.  The kernels therefore need
// only the K-th largest key t (a radix select, eight 8-bit digits from the
// top) and count per request the keys >= t; no sort.
struct BudgetLds {
  uint64_t keys[SV_MAX_BUDGET_POSITIONS];
  int32_t counts[SV_MAX_BUDGET_POSITIONS];
  int32_t hist[256];
  float red[kBudgetWaves];
  int32_t wtot[kBudgetWaves];
  int32_t s_valid, s_need, s_whole;
  uint64_t s_prefix;
  uint64_t s_min[kBudgetWaves];
};

// Prefix-confidence products and keys; returns this thread's share of the
// sum of all scores.  Leaves the keys in registers (key[j] = slot
// j * kBudgetThreads + tid) and the number of valid positions in s_valid.
__device__ float build_keys(const float* conf, int32_t B, int32_t D, const int32_t* max_depth,
                            BudgetLds& S, uint64_t (&key)[kKeySlots]) {
  const int tid = threadIdx.x;
  const int N = B * D;
  for (int r = tid; r < B; r += kBudgetThreads) S.counts[r] = 0;
  if (tid == 0) S.s_valid = 0;
  // One coalesced pass stages the confidences in the key slots (as float
  // bits); the product loop then reads LDS.
  for (int i = tid; i < N; i += kBudgetThreads) S.keys[i] = (uint64_t)__float_as_uint(conf[i]);
  __syncthreads();

  // Prefix-confidence products, left to right in float32, one request per
  // thread; each slot is read and then overwritten by the same thread, eight
  // positions at a time (the eight reads issued together).
  int valid = 0;
  float total = 0.0f;
  for (int r = tid; r < B; r += kBudgetThreads) {
    int lim = max_depth ? max_depth[r] : D;
    lim = lim < 0 ? 0 : (lim > D ? D : lim);
    float sc = 1.0f;
    for (int k0 = 0; k0 < D; k0 += 8) {
      float cv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        cv[j] = (k0 + j < lim) ? __uint_as_float((uint32_t)S.keys[r * D + k0 + j]) : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = k0 + j;
        if (k >= D) break;
        const int idx = r * D + k;
        if (k >= lim) {  // past this request's limit: key 0, never kept
          S.keys[idx] = 0ull;
          continue;
        }
        float c = cv[j];
        if (!(c >= 0.0f)) c = 0.0f;  // NaN and negatives read as 0
        if (c > 1.0f) c = 1.0f;
        sc = sc * c;
        total += sc;
        S.keys[idx] = ((uint64_t)__float_as_uint(sc) << 32) | (uint64_t)(~(uint32_t)idx);
      }
    }
    valid += lim;
  }
  // one LDS atomic per wavefront (the wavefront's total), not per thread
  for (int m = 1; m < kWave; m <<= 1) valid += __shfl_xor(valid, m);
  if ((tid & (kWave - 1)) == 0 && valid) atomicAdd(&S.s_valid, valid);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int i = j * kBudgetThreads + tid;
    key[j] = i < N ? S.keys[i] : 0ull;
  }
  return total;
}

// The Keff-th largest key (~0 when Keff == 0: nothing kept).  After digit
// round d, s_prefix holds its top 8 (d + 1) bits and s_need its rank among
// the keys that share them.  When every key sharing the prefix is kept
// (s_need equals their count), the threshold is the smallest of them and the
// remaining rounds are skipped.
__device__ uint64_t select_threshold(const uint64_t (&key)[kKeySlots], int N, int32_t Keff,
                                     BudgetLds& S) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  __syncthreads();  // every thread is done with the previous call's state
  if (tid == 0) {
    S.s_prefix = 0ull;
    S.s_need = Keff;
    S.s_whole = 0;
  }
  if (Keff <= 0) return ~0ull;
  if (Keff >= S.s_valid) return 1ull;  // every valid position is kept (their keys are >= 1)
  for (int d = 0; d < 8; ++d) {
    const int shift = 56 - 8 * d;
    if (tid < 256) S.hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = S.s_prefix;
    const int32_t need = S.s_need;
#pragma unroll
    for (int j = 0; j < kKeySlots; ++j) {
      // keys sharing the selected top bits (all keys for the first digit)
      const bool match = d == 0 || (key[j] >> (shift + 8)) == (prefix >> (shift + 8));
      if (match && j * kBudgetThreads + tid < N)
        atomicAdd(&S.hist[(int)((key[j] >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 255 - 4 l .. 252 - 4 l (descending)
      int32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = S.hist[255 - 4 * lane - j];
      const int32_t sum = h[0] + h[1] + h[2] + h[3];
      const int32_t incl = wave_incl_scan(sum);
      int32_t run = incl - sum;
      if (run < need && need <= incl) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < need && need <= run + h[j]) {
            S.s_prefix = prefix | ((uint64_t)(255 - 4 * lane - j) << shift);
            S.s_need = need - run;
            S.s_whole = (need - run == h[j]) ? 1 : 0;
          }
          run += h[j];
        }
      }
    }
    __syncthreads();
    if (S.s_whole && d < 7) {
      // smallest key among those sharing the selected top 8 (d + 1) bits
      const uint64_t pre = S.s_prefix;
      uint64_t mn = ~0ull;
#pragma unroll
      for (int j = 0; j < kKeySlots; ++j)
        if (j * kBudgetThreads + tid < N && (key[j] >> shift) == (pre >> shift) && key[j] < mn)
          mn = key[j];
      for (int m = 1; m < kWave; m <<= 1) {
        const uint32_t lo32 = __shfl_xor((uint32_t)(mn & 0xffffffffull), m);
        const uint32_t hi32 = __shfl_xor((uint32_t)(mn >> 32), m);
        const uint64_t o = ((uint64_t)hi32 << 32) | lo32;
        mn = o < mn ? o : mn;
      }
      if (lane == 0) S.s_min[wave] = mn;
      __syncthreads();
      uint64_t t = S.s_min[0];
      for (int w2 = 1; w2 < kBudgetWaves; ++w2) t = S.s_min[w2] < t ? S.s_min[w2] : t;
      S.s_prefix = t;  // every thread writes the same value
      __syncthreads();
      break;
    }
  }
  return S.s_prefix;
}

// Kept positions per request (counts), the kept utility (block sum) and the
// packed row offsets: exclusive scans of c_r (draft rows) and c_r + 1
// (target rows) over the requests; thread t takes kKeySlots consecutive
// requests.
__device__ float write_allocation(const uint64_t (&key)[kKeySlots], int32_t B, int32_t D,
                                  uint64_t thr, BudgetLds& S, int32_t* depth,
                                  int64_t* draft_row0, int64_t* target_row0) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int N = B * D;
  float kept = 0.0f;
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int i = j * kBudgetThreads + tid;
    if (i < N && key[j] != 0ull && key[j] >= thr) {
      atomicAdd(&S.counts[i / D], 1);
      kept += __uint_as_float((uint32_t)(key[j] >> 32));
    }
  }
  __syncthreads();
  kept = block_sum_budget(kept, S.red);
  int32_t c[kKeySlots];
  int32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int r = tid * kKeySlots + j;
    c[j] = r < B ? S.counts[r] : 0;
    mine += c[j];
  }
  const int32_t wincl = wave_incl_scan(mine);
  if (lane == kWave - 1) S.wtot[wave] = wincl;
  __syncthreads();
  int32_t before = wincl - mine;
  for (int w = 0; w < wave; ++w) before += S.wtot[w];
  int64_t dr = before;
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int r = tid * kKeySlots + j;
    if (r < B) {
      depth[r] = c[j];
      if (draft_row0) draft_row0[r] = dr;
      if (target_row0) target_row0[r] = dr + r;
    }
    dr += c[j];
  }
  return kept;
}

__global__ __launch_bounds__(kBudgetThreads) void k_budget(const float* conf, int32_t B, int32_t D,
                                                           const int32_t* max_depth, int64_t K,
                                                           int32_t* depth, int64_t* draft_row0,
                                                           int64_t* target_row0, float* utility) {
  __shared__ BudgetLds S;
  uint64_t key[kKeySlots];
  float total = build_keys(conf, B, D, max_depth, S, key);
  int64_t kk = K < 0 ? 0 : K;
  if (kk > S.s_valid) kk = S.s_valid;
  const uint64_t thr = select_threshold(key, B * D, (int32_t)kk, S);
  const float kept = write_allocation(key, B, D, thr, S, depth, draft_row0, target_row0);
  total = block_sum_budget(total, S.red);
  if (utility && threadIdx.x == 0) {
    utility[0] = kept;
    utility[1] = total;
  }
}

hipError_t launch_budget(const float* conf, int32_t B, int32_t D, const int32_t* max_depth,
                         int64_t K, int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                         float* utility, hipStream_t stream) {
  hipLaunchKernelGGL(k_budget, dim3(1), dim3(kBudgetThreads), 0, stream, conf, B, D, max_depth, K,
                     depth, draft_row0, target_row0, utility);
  return hipGetLastError();
}

// The fixed-depth baseline of the budget widget ("AngelSpec: specialize the
// drafter...", section "D-cut"): the same K positions spread evenly, depth
// floor(K / B) for every request and one more for the first K mod B, never
// past D_max.  Scores, the kept utility and the row offsets as k_budget
// writes them, so that the two allocations' retained utility compare.
__global__ __launch_bounds__(kBudgetThreads) void k_budget_fixed(const float* conf, int32_t B,
                                                                 int32_t D, int64_t K,
                                                                 int32_t* depth,
                                                                 int64_t* draft_row0,
                                                                 int64_t* target_row0,
                                                                 float* utility) {
  __shared__ BudgetLds S;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  uint64_t key[kKeySlots];
  float total = build_keys(conf, B, D, nullptr, S, key);
  const int64_t kk = K < 0 ? 0 : K;
  const int64_t base = kk / B, extra = kk % B;
  auto fixed = [&](int r) {
    const int64_t n = base + (r < extra ? 1 : 0);
    return (int32_t)(n > D ? D : n);
  };
  float kept = 0.0f;
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int i = j * kBudgetThreads + tid;
    if (i < B * D && (i % D) < fixed(i / D)) kept += __uint_as_float((uint32_t)(key[j] >> 32));
  }
  kept = block_sum_budget(kept, S.red);
  total = block_sum_budget(total, S.red);
  // row offsets: exclusive scans of n_r and n_r + 1 over the requests, thread
  // t taking kKeySlots consecutive requests
  int32_t c[kKeySlots];
  int32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int r = tid * kKeySlots + j;
    c[j] = r < B ? fixed(r) : 0;
    mine += c[j];
  }
  const int32_t wincl = wave_incl_scan(mine);
  if (lane == kWave - 1) S.wtot[wave] = wincl;
  __syncthreads();
  int32_t before = wincl - mine;
  for (int w = 0; w < wave; ++w) before += S.wtot[w];
  int64_t dr = before;
#pragma unroll
  for (int j = 0; j < kKeySlots; ++j) {
    const int r = tid * kKeySlots + j;
    if (r < B) {
      depth[r] = c[j];
      if (draft_row0) draft_row0[r] = dr;
      if (target_row0) target_row0[r] = dr + r;
    }
    dr += c[j];
  }
  if (utility && tid == 0) {
    utility[0] = kept;
    utility[1] = total;
  }
}

hipError_t launch_budget_fixed(const float* conf, int32_t B, int32_t D, int64_t K, int32_t* depth,
                               int64_t* draft_row0, int64_t* target_row0, float* utility,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_budget_fixed, dim3(1), dim3(kBudgetThreads), 0, stream, conf, B, D, K,
                     depth, draft_row0, target_row0, utility);
  return hipGetLastError();
}

// D-cut's keep ratio ("AngelSpec: specialize the drafter...", section
// "D-cut": the ratio is picked each step from a few values by a runtime
// cost table so as to maximise projected throughput, not kept length).
// Ratio j keeps K_j = ceil(rho_j N) of the N drafted positions; its
// projected tokens are B (one per request) plus the kept utility U_j (the
// sum of the kept prefix-confidence products, equation A-hat over the
// batch), divided by the latency the caller's table gives this batch size.
// The first ratio with the largest value wins; its allocation is written
// as by k_budget.
__global__ __launch_bounds__(kBudgetThreads) void k_budget_ratio(
    const float* conf, int32_t B, int32_t D, const int32_t* max_depth, RatioArgs ra,
    int32_t* choice, int64_t* K_chosen, float* projected, int32_t* depth, int64_t* draft_row0,
    int64_t* target_row0, float* utility) {
  __shared__ BudgetLds S;
  const int tid = threadIdx.x;
  const int N = B * D;
  uint64_t key[kKeySlots];
  float total = build_keys(conf, B, D, max_depth, S, key);
  const int64_t valid = S.s_valid;
  int best = -1;
  double best_tp = 0.0;
  uint64_t best_thr = ~0ull;
  int64_t best_K = 0;
  for (int j = 0; j < ra.n; ++j) {
    int64_t Kj = (int64_t)ceil(ra.ratio[j] * (double)valid);
    if (Kj > valid) Kj = valid;
    const uint64_t thr = select_threshold(key, N, (int32_t)Kj, S);
    float kept = 0.0f;
#pragma unroll
    for (int s = 0; s < kKeySlots; ++s) {
      const int i = s * kBudgetThreads + tid;
      if (i < N && key[s] != 0ull && key[s] >= thr) kept += __uint_as_float((uint32_t)(key[s] >> 32));
    }
    kept = block_sum_budget(kept, S.red);
    const double tp = ((double)B + (double)kept) / ra.latency[j];
    if (projected && tid == 0) projected[j] = (float)tp;
    if (best < 0 || tp > best_tp) {  // block-uniform values: every thread agrees
      best = j;
      best_tp = tp;
      best_thr = thr;
      best_K = Kj;
    }
  }
  const float kept = write_allocation(key, B, D, best_thr, S, depth, draft_row0, target_row0);
  total = block_sum_budget(total, S.red);
  if (tid == 0) {
    *choice = best;
    *K_chosen = best_K;
    if (utility) {
      utility[0] = kept;
      utility[1] = total;
    }
  }
}

hipError_t launch_budget_ratio(const float* conf, int32_t B, int32_t D, const int32_t* max_depth,
                               const RatioArgs& ra, int32_t* choice, int64_t* K_chosen,
                               float* projected, int32_t* depth, int64_t* draft_row0,
                               int64_t* target_row0, float* utility, hipStream_t stream) {
  hipLaunchKernelGGL(k_budget_ratio, dim3(1), dim3(kBudgetThreads), 0, stream, conf, B, D,
                     max_depth, ra, choice, K_chosen, projected, depth, draft_row0, target_row0,
                     utility);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Acceptance statistics of one batch (sv_stats.hpp): one workgroup of 16
// wavefronts, four requests of each wavefront loaded together.
constexpr int kStatsThreads = 1024;
constexpr int kStatsWaves = kStatsThreads / kWave;

__global__ __launch_bounds__(kStatsThreads) void k_accept_stats(
    const int32_t* depth, const float* alpha, const int32_t* accepted_len, int32_t B, int32_t D,
    float* expected_len, float* per_depth, float* summary) {
  __shared__ StatsLds S;
  accept_stats_block<kStatsWaves, 4>(depth, alpha, accepted_len, B, D, expected_len, per_depth,
                                     summary, S);
}

// Statistics over many verified batches (the decode loop's steps; MAL,
// mean acceptance and position-wise acceptance over whole generations, as
// the tradepoint.io page, "The MTP path", reports them).  One workgroup adds
// one batch to the caller's running totals (float64, so counts stay exact
// to 2^53) and writes the summary of the new totals.  Layout of accum:
// [0] tokens emitted (sum of tau + 1), [1] requests, [2] sum of E[tau],
// [3 + k] requests with depth > k, [3 + D + k] requests with tau > k.
__global__ __launch_bounds__(kStatsThreads) void k_accept_accumulate(
    const int32_t* depth, const float* alpha, const int32_t* accepted_len, int32_t B, int32_t D,
    double* accum, float* summary) {
  __shared__ int32_t s_ver[kStatsWaves][kWave];
  __shared__ int32_t s_acc[kStatsWaves][kWave];
  __shared__ double s_e[kStatsWaves];
  __shared__ int64_t s_emit[kStatsWaves];
  __shared__ double s_tot[3 + 2 * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int32_t ver = 0, acc = 0;
  double esum = 0.0;  // lane 0
  int64_t emit = 0;   // lane 0
  for (int r = wave; r < B; r += kStatsWaves) {
    int n = depth[r];
    const int tau = accepted_len[r];
    const float a_raw = (alpha && lane < D) ? alpha[(int64_t)r * D + lane] : 1.0f;
    n = n < 0 ? 0 : (n > D ? D : n);
    if (lane < n) ver += 1;
    if (lane < D && tau > lane) acc += 1;
    if (alpha) {
      const bool in = lane < n;
      float pref = in ? a_raw : 1.0f;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const float o = __shfl_up(pref, d);
        if (lane >= d) pref *= o;
      }
      const float e = wave_sum(in ? pref : 0.0f);
      esum += (double)e;
    }
    emit += tau + 1;
  }
  s_ver[wave][lane] = ver;
  s_acc[wave][lane] = acc;
  if (lane == 0) {
    s_e[wave] = esum;
    s_emit[wave] = emit;
  }
  __syncthreads();
  if (wave == 0) {
    if (lane < D) {
      int32_t v = 0, a = 0;
      for (int w = 0; w < kStatsWaves; ++w) {
        v += s_ver[w][lane];
        a += s_acc[w][lane];
      }
      const double tv = accum[3 + lane] + (double)v;
      const double ta = accum[3 + D + lane] + (double)a;
      accum[3 + lane] = tv;
      accum[3 + D + lane] = ta;
      s_tot[3 + lane] = tv;
      s_tot[3 + D + lane] = ta;
    }
    if (lane == 0) {
      double e = 0.0;
      int64_t m = 0;
      for (int w = 0; w < kStatsWaves; ++w) {
        e += s_e[w];
        m += s_emit[w];
      }
      const double t0 = accum[0] + (double)m, t1 = accum[1] + (double)B, t2 = accum[2] + e;
      accum[0] = t0;
      accum[1] = t1;
      accum[2] = t2;
      s_tot[0] = t0;
      s_tot[1] = t1;
      s_tot[2] = t2;
    }
  }
  __syncthreads();
  if (summary && wave == 0) {
    const double req = s_tot[1];
    if (lane < D) summary[3 + lane] = req > 0.0 ? (float)(s_tot[3 + D + lane] / req) : 0.0f;
    if (lane == 0) {
      double sum_n = 0.0;
      for (int k = 0; k < D; ++k) sum_n += s_tot[3 + k];
      summary[0] = req > 0.0 ? (float)(s_tot[0] / req) : 0.0f;
      summary[1] = req > 0.0 ? (float)(1.0 + s_tot[2] / req) : 0.0f;
      summary[2] = sum_n > 0.0 ? (float)((s_tot[0] - req) / sum_n) : 0.0f;
    }
  }
}

hipError_t launch_accumulate(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                             int32_t B, int32_t D, double* accum, float* summary,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_accept_accumulate, dim3(1), dim3(kStatsThreads), 0, stream, depth, alpha,
                     accepted_len, B, D, accum, summary);
  return hipGetLastError();
}

hipError_t launch_stats(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                        int32_t B, int32_t D, float* expected_len, float* per_depth,
                        float* summary, hipStream_t stream) {
  hipLaunchKernelGGL(k_accept_stats, dim3(1), dim3(kStatsThreads), 0, stream, depth, alpha,
                     accepted_len, B, D, expected_len, per_depth, summary);
  return hipGetLastError();
}

}  // namespace sv
