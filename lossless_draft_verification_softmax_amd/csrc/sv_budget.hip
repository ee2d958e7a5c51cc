// sv_budget.hip -- the batch-shared verification budget ("AngelSpec:
// specialize the drafter...", section "D-cut": Figure 3 flattens every draft
// position of the batch, sorts by confidence and keeps a global top-K;
// equation A-hat scores a request's kept prefix by its prefix-confidence
// products).
//
// One workgroup of 1024 threads: float32 prefix products, 64-bit keys
// (score bits above the complemented flat index, so equal scores order by
// lower request, then lower position), a bitonic sort in LDS, then per-request
// counts and the packed row offsets.  The whole batch (B * D_max <= 4096
// keys, 32 KB) stays in LDS; B <= 4096.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

constexpr int kBudgetThreads = 1024;

__device__ __forceinline__ float block_sum_budget(float v, float* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < kBudgetThreads / kWave; ++w) t += lds[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kBudgetThreads) void k_budget(const float* conf, int32_t B, int32_t D,
                                                           const int32_t* max_depth, int64_t K,
                                                           int32_t N2, int32_t* depth,
                                                           int64_t* draft_row0, int64_t* target_row0,
                                                           float* utility) {
  __shared__ uint64_t keys[SV_MAX_BUDGET_POSITIONS];
  __shared__ int32_t counts[SV_MAX_BUDGET_POSITIONS];
  __shared__ float red[kBudgetThreads / kWave];
  __shared__ int32_t s_valid;
  const int tid = threadIdx.x;
  const int N = B * D;
  for (int i = tid; i < N2; i += kBudgetThreads) keys[i] = 0ull;
  for (int r = tid; r < B; r += kBudgetThreads) counts[r] = 0;
  if (tid == 0) s_valid = 0;
  __syncthreads();

  // Prefix-confidence products, left to right in float32.
  int valid = 0;
  float total = 0.0f;
  for (int r = tid; r < B; r += kBudgetThreads) {
    int lim = max_depth ? max_depth[r] : D;
    lim = lim < 0 ? 0 : (lim > D ? D : lim);
    float s = 1.0f;
    for (int k = 0; k < lim; ++k) {
      const int idx = r * D + k;
      float c = conf[idx];
      if (!(c >= 0.0f)) c = 0.0f;  // NaN and negatives read as 0
      if (c > 1.0f) c = 1.0f;
      s = s * c;
      total += s;
      keys[idx] = ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(~(uint32_t)idx);
    }
    valid += lim;
  }
  atomicAdd(&s_valid, valid);
  __syncthreads();

  // Bitonic sort, descending.  Padding and cut-off positions hold key 0,
  // below every real key (a real key's low word ~idx is never 0).
  for (int size = 2; size <= N2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < N2 / 2; i += kBudgetThreads) {
        const int a = (i / stride) * 2 * stride + (i % stride);
        const int b = a + stride;
        const bool desc = (a & size) == 0;
        const uint64_t ka = keys[a], kb = keys[b];
        if (desc ? (ka < kb) : (ka > kb)) {
          keys[a] = kb;
          keys[b] = ka;
        }
      }
      __syncthreads();
    }
  }

  int64_t kk = K < 0 ? 0 : K;
  if (kk > s_valid) kk = s_valid;
  const int Keff = (int)kk;
  float kept = 0.0f;
  for (int i = tid; i < Keff; i += kBudgetThreads) {
    const uint32_t idx = ~(uint32_t)(keys[i] & 0xffffffffull);
    atomicAdd(&counts[idx / D], 1);
    kept += __uint_as_float((uint32_t)(keys[i] >> 32));
  }
  __syncthreads();
  kept = block_sum_budget(kept, red);
  total = block_sum_budget(total, red);

  if (tid == 0) {
    int64_t dr = 0, tr = 0;
    for (int r = 0; r < B; ++r) {
      const int32_t c = counts[r];
      depth[r] = c;
      if (draft_row0) draft_row0[r] = dr;
      if (target_row0) target_row0[r] = tr;
      dr += c;
      tr += c + 1;
    }
    if (utility) {
      utility[0] = kept;
      utility[1] = total;
    }
  }
}

hipError_t launch_budget(const float* conf, int32_t B, int32_t D, const int32_t* max_depth,
                         int64_t K, int32_t* depth, int64_t* draft_row0, int64_t* target_row0,
                         float* utility, hipStream_t stream) {
  int32_t N = B * D, N2 = 2;
  while (N2 < N) N2 <<= 1;
  hipLaunchKernelGGL(k_budget, dim3(1), dim3(kBudgetThreads), 0, stream, conf, B, D, max_depth, K,
                     N2, depth, draft_row0, target_row0, utility);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Acceptance statistics (equation L_e2e of "AngelSpec: specialize the
// drafter...", section "MTP"; MAL and mean acceptance of the tradepoint.io
// page, "The MTP path").  One workgroup; fixed summation orders.
constexpr int kStatsThreads = 256;

__global__ __launch_bounds__(kStatsThreads) void k_accept_stats(
    const int32_t* depth, const float* alpha, const int32_t* accepted_len, int32_t B, int32_t D,
    float* expected_len, float* per_depth, float* summary) {
  const int tid = threadIdx.x;
  for (int r = tid; r < B; r += kStatsThreads) {
    int n = depth[r];
    n = n < 0 ? 0 : (n > D ? D : n);
    float e = 0.0f, pref = 1.0f;
    if (alpha)
      for (int k = 0; k < n; ++k) {
        pref *= alpha[(int64_t)r * D + k];
        e += pref;
      }
    if (expected_len) expected_len[r] = e;
  }
  if (per_depth) {
    for (int k = tid; k < D; k += kStatsThreads) {
      float tested = 0.0f, kept = 0.0f, asum = 0.0f;
      int with_k = 0;
      for (int r = 0; r < B; ++r) {
        int n = depth[r];
        n = n < 0 ? 0 : (n > D ? D : n);
        if (k >= n) continue;
        const int tau = accepted_len[r];
        ++with_k;
        if (tau >= k) tested += 1.0f;
        if (tau > k) kept += 1.0f;
        if (alpha) asum += alpha[(int64_t)r * D + k];
      }
      per_depth[k] = tested;
      per_depth[D + k] = kept;
      per_depth[2 * D + k] = with_k ? asum / (float)with_k : 0.0f;
    }
  }
  if (summary && tid == 0) {
    float st = 0.0f, sn = 0.0f, se = 0.0f;
    for (int r = 0; r < B; ++r) {
      int n = depth[r];
      n = n < 0 ? 0 : (n > D ? D : n);
      st += (float)accepted_len[r];
      sn += (float)n;
      if (alpha) {
        float e = 0.0f, pref = 1.0f;
        for (int k = 0; k < n; ++k) {
          pref *= alpha[(int64_t)r * D + k];
          e += pref;
        }
        se += e;
      }
    }
    summary[0] = B ? 1.0f + st / (float)B : 0.0f;
    summary[1] = B ? 1.0f + se / (float)B : 0.0f;
    summary[2] = sn > 0.0f ? st / sn : 0.0f;
    summary[3] = sn;
  }
}

hipError_t launch_stats(const int32_t* depth, const float* alpha, const int32_t* accepted_len,
                        int32_t B, int32_t D, float* expected_len, float* per_depth,
                        float* summary, hipStream_t stream) {
  hipLaunchKernelGGL(k_accept_stats, dim3(1), dim3(kStatsThreads), 0, stream, depth, alpha,
                     accepted_len, B, D, expected_len, per_depth, summary);
  return hipGetLastError();
}

}  // namespace sv
