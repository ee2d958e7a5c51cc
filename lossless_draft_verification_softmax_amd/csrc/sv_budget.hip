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
  // One coalesced pass stages the confidences in the key slots (as float
  // bits); the product loop below then reads LDS instead of waiting on one
  // global load per position.  Each slot is read and then overwritten by
  // the same thread.
  for (int i = tid; i < N; i += kBudgetThreads) keys[i] = (uint64_t)__float_as_uint(conf[i]);
  __syncthreads();

  // Prefix-confidence products, left to right in float32.
  int valid = 0;
  float total = 0.0f;
  for (int r = tid; r < B; r += kBudgetThreads) {
    int lim = max_depth ? max_depth[r] : D;
    lim = lim < 0 ? 0 : (lim > D ? D : lim);
    float s = 1.0f;
    for (int k = 0; k < D; ++k) {
      const int idx = r * D + k;
      if (k >= lim) {  // past this request's limit: key 0, never kept
        keys[idx] = 0ull;
        continue;
      }
      float c = __uint_as_float((uint32_t)keys[idx]);
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

  // Bitonic sort, descending, over N2 (a power of two, >= 64) keys.  Key i
  // lives in register slot i / 1024 of thread i % 1024.  Partners at stride
  // >= 1024 are in the same thread, strides 64..512 go through LDS, strides
  // below 64 stay inside the wavefront (shuffles, no barrier).  Padding and
  // cut-off positions hold key 0, below every real key (a real key's low
  // word ~idx is never 0).
  constexpr int kSlots = SV_MAX_BUDGET_POSITIONS / kBudgetThreads;
  const int nslots = (N2 + kBudgetThreads - 1) / kBudgetThreads;
  uint64_t key[kSlots];
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl) {
    const int i = sl * kBudgetThreads + tid;
    key[sl] = (sl < nslots && i < N2) ? keys[i] : 0ull;
  }
  for (int size = 2; size <= N2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= kBudgetThreads) {
        const int sx = stride / kBudgetThreads;
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
          if (sl >= nslots || (sl & sx)) continue;
          const int i = sl * kBudgetThreads + tid;
          const bool desc = (i & size) == 0;
#pragma unroll
          for (int sh = 0; sh < kSlots; ++sh) {
            if (sh != (sl ^ sx)) continue;
            const uint64_t a = key[sl], b = key[sh];
            const bool swap = desc ? (a < b) : (a > b);
            key[sl] = swap ? b : a;
            key[sh] = swap ? a : b;
          }
        }
      } else if (stride >= kWave) {
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl)
          if (sl < nslots) keys[sl * kBudgetThreads + tid] = key[sl];
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
          if (sl >= nslots) continue;
          const int i = sl * kBudgetThreads + tid;
          if (i >= N2) continue;
          const int pi = i ^ stride;
          const uint64_t other = keys[pi];
          const bool desc = (i & size) == 0;
          const bool lower = i < pi;
          const uint64_t hi = key[sl] > other ? key[sl] : other;
          const uint64_t lo = key[sl] > other ? other : key[sl];
          key[sl] = (lower == desc) ? hi : lo;
        }
        __syncthreads();
      } else {
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
          if (sl >= nslots) continue;
          const int i = sl * kBudgetThreads + tid;
          const uint32_t lo32 = __shfl_xor((uint32_t)(key[sl] & 0xffffffffull), stride);
          const uint32_t hi32 = __shfl_xor((uint32_t)(key[sl] >> 32), stride);
          const uint64_t other = ((uint64_t)hi32 << 32) | lo32;
          const bool desc = (i & size) == 0;
          const bool lower = (i & stride) == 0;
          const uint64_t hi = key[sl] > other ? key[sl] : other;
          const uint64_t lo = key[sl] > other ? other : key[sl];
          key[sl] = (lower == desc) ? hi : lo;
        }
      }
    }
  }
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl)
    if (sl < nslots && sl * kBudgetThreads + tid < N2) keys[sl * kBudgetThreads + tid] = key[sl];
  __syncthreads();

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
  int32_t N = B * D, N2 = kWave;  // at least one full wavefront of keys
  while (N2 < N) N2 <<= 1;
  hipLaunchKernelGGL(k_budget, dim3(1), dim3(kBudgetThreads), 0, stream, conf, B, D, max_depth, K,
                     N2, depth, draft_row0, target_row0, utility);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Acceptance statistics (equation L_e2e of "AngelSpec: specialize the
// drafter...", section "MTP"; MAL and mean acceptance of the tradepoint.io
// page, "The MTP path").  One workgroup of 16 wavefronts; wavefront w takes
// requests w, w + 16, ...: lane k holds position k (D_max <= 64), a
// wavefront prefix product gives prod_{j<=k} alpha_j and a wavefront sum
// gives E[tau_r].  Per-depth counters stay in the lanes; the 16 wavefront
// partials are then added in a fixed order.
constexpr int kStatsThreads = 1024;
constexpr int kStatsWaves = kStatsThreads / kWave;

__global__ __launch_bounds__(kStatsThreads) void k_accept_stats(
    const int32_t* depth, const float* alpha, const int32_t* accepted_len, int32_t B, int32_t D,
    float* expected_len, float* per_depth, float* summary) {
  __shared__ float s_tested[kStatsWaves][kWave];
  __shared__ float s_kept[kStatsWaves][kWave];
  __shared__ float s_asum[kStatsWaves][kWave];
  __shared__ int32_t s_with[kStatsWaves][kWave];
  __shared__ float s_sum[kStatsWaves][3];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float tested = 0.0f, kept = 0.0f, asum = 0.0f;
  int32_t with_k = 0;
  float st = 0.0f, sn = 0.0f, se = 0.0f;  // lane 0 only
  for (int r = wave; r < B; r += kStatsWaves) {
    int n = depth[r];
    n = n < 0 ? 0 : (n > D ? D : n);
    const int tau = accepted_len[r];
    const bool in = lane < n;
    const float a = (in && alpha) ? alpha[(int64_t)r * D + lane] : 1.0f;
    // inclusive prefix product over lanes (fixed Hillis-Steele order)
    float pref = a;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const float o = __shfl_up(pref, d);
      if (lane >= d) pref *= o;
    }
    const float e = wave_sum((in && alpha) ? pref : 0.0f);
    if (in) {
      with_k += 1;
      if (tau >= lane) tested += 1.0f;
      if (tau > lane) kept += 1.0f;
      if (alpha) asum += a;
    }
    if (lane == 0) {
      if (expected_len) expected_len[r] = e;
      st += (float)tau;
      sn += (float)n;
      se += e;
    }
  }
  s_tested[wave][lane] = tested;
  s_kept[wave][lane] = kept;
  s_asum[wave][lane] = asum;
  s_with[wave][lane] = with_k;
  if (lane == 0) {
    s_sum[wave][0] = st;
    s_sum[wave][1] = sn;
    s_sum[wave][2] = se;
  }
  __syncthreads();
  if (per_depth && wave == 0 && lane < D) {
    float t = 0.0f, k = 0.0f, a = 0.0f;
    int32_t w = 0;
    for (int v = 0; v < kStatsWaves; ++v) {
      t += s_tested[v][lane];
      k += s_kept[v][lane];
      a += s_asum[v][lane];
      w += s_with[v][lane];
    }
    per_depth[lane] = t;
    per_depth[D + lane] = k;
    per_depth[2 * D + lane] = w ? a / (float)w : 0.0f;
  }
  if (summary && threadIdx.x == 0) {
    float t = 0.0f, n = 0.0f, e = 0.0f;
    for (int v = 0; v < kStatsWaves; ++v) {
      t += s_sum[v][0];
      n += s_sum[v][1];
      e += s_sum[v][2];
    }
    summary[0] = B ? 1.0f + t / (float)B : 0.0f;
    summary[1] = B ? 1.0f + e / (float)B : 0.0f;
    summary[2] = n > 0.0f ? t / n : 0.0f;
    summary[3] = n;
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
