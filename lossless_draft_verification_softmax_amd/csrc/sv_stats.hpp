// sv_stats.hpp -- acceptance statistics of one verified batch (equation
// L_e2e of "AngelSpec: specialize the drafter...", section "MTP"; MAL and
// mean acceptance of the tradepoint.io page, "The MTP path") as the routine
// of one workgroup.  The statistics kernel runs it with 16 wavefronts; the
// float64 tile pass runs it with its 4 on one extra workgroup, beside its
// tiles, so that a verification call can leave the statistics of its own
// batch without a launch of its own.
//
// Lane k of a wavefront holds position k (D_max <= 64): a wavefront prefix
// product gives prod_{j<=k} alpha_j and a wavefront sum gives E[tau_r].
// Requests are dealt to 16 virtual wavefronts (request r to r mod 16), each
// of which adds its requests in increasing order; the 16 partials are then
// added in a fixed order.  A workgroup of W wavefronts runs 16 / W virtual
// wavefronts in each, so every workgroup size gives the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.hpp"

namespace sv {

constexpr int kStatsVirtualWaves = 16;

struct StatsLds {
  float tested[kStatsVirtualWaves][kWave];
  float kept[kStatsVirtualWaves][kWave];
  float asum[kStatsVirtualWaves][kWave];
  int32_t with[kStatsVirtualWaves][kWave];
  float sum[kStatsVirtualWaves][3];
};

// Inclusive prefix product over the lanes below D (lanes at or past D are
// never used), in the Hillis-Steele order: at step d lane k >= d multiplies
// in lane k - d's product of the step before.  With D <= 16 only the first
// row of 16 lanes matters, and row shifts (DPP) carry the steps; otherwise
// lane permutes over the wavefront, stopping once d reaches D.  The same
// products in the same order either way.
__device__ __forceinline__ float lane_prefix_product(float a, int D) {
  const int lane = threadIdx.x & (kWave - 1);
  float pref = a;
  if (D <= 16) {
    const int r = lane & 15;
    float o = dpp_f<0x111>(pref);  // row_shr:1
    if (r >= 1) pref *= o;
    o = dpp_f<0x112>(pref);        // row_shr:2
    if (r >= 2) pref *= o;
    o = dpp_f<0x114>(pref);        // row_shr:4
    if (r >= 4) pref *= o;
    o = dpp_f<0x118>(pref);        // row_shr:8
    if (r >= 8) pref *= o;
    return pref;
  }
  for (int d = 1; d < D && d < kWave; d <<= 1) {  // uniform
    const float o = __shfl_up(pref, d);
    if (lane >= d) pref *= o;
  }
  return pref;
}

// W wavefronts in the workgroup; BATCH requests of each virtual wavefront
// have their depths, accepted lengths and acceptance rates (all D positions,
// whatever the depth) loaded together.  Every thread of the workgroup calls
// it; it ends with the outputs written (no barrier after the last write).
template <int W, int BATCH>
__device__ __forceinline__ void accept_stats_block(const int32_t* depth, const float* alpha,
                                                   const int32_t* accepted_len, int32_t B,
                                                   int32_t D, float* expected_len,
                                                   float* per_depth, float* summary,
                                                   StatsLds& S) {
  constexpr int R = kStatsVirtualWaves / W;
  static_assert(R * W == kStatsVirtualWaves, "wavefronts must divide 16");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float tested[R], kept[R], asum[R], st[R], sn[R], se[R];  // st, sn, se: lane 0 only
  int32_t with_k[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    tested[j] = kept[j] = asum[j] = st[j] = sn[j] = se[j] = 0.0f;
    with_k[j] = 0;
  }
  // Virtual wavefront v = wave + j W takes requests v, v + 16, ...
  for (int r0 = wave; r0 < B; r0 += kStatsVirtualWaves * BATCH) {
    int nb[BATCH][R], taub[BATCH][R];
    float ab[BATCH][R];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int r = r0 + i * kStatsVirtualWaves + j * W;
        nb[i][j] = 0;
        taub[i][j] = 0;
        ab[i][j] = 1.0f;
        if (r < B) {
          nb[i][j] = depth[r];
          taub[i][j] = accepted_len[r];
          if (alpha && lane < D) ab[i][j] = alpha[(int64_t)r * D + lane];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int r = r0 + i * kStatsVirtualWaves + j * W;
        if (r >= B) continue;  // uniform
        int n = nb[i][j];
        const int tau = taub[i][j];
        n = n < 0 ? 0 : (n > D ? D : n);
        const bool in = lane < n;
        const float a = (in && alpha) ? ab[i][j] : 1.0f;
        const float pref = lane_prefix_product(a, D);
        const float e = wave_sum((in && alpha) ? pref : 0.0f);
        if (in) {
          with_k[j] += 1;
          if (tau >= lane) tested[j] += 1.0f;
          if (tau > lane) kept[j] += 1.0f;
          if (alpha) asum[j] += a;
        }
        if (lane == 0) {
          if (expected_len) expected_len[r] = e;
          st[j] += (float)tau;
          sn[j] += (float)n;
          se[j] += e;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int v = wave + j * W;
    S.tested[v][lane] = tested[j];
    S.kept[v][lane] = kept[j];
    S.asum[v][lane] = asum[j];
    S.with[v][lane] = with_k[j];
    if (lane == 0) {
      S.sum[v][0] = st[j];
      S.sum[v][1] = sn[j];
      S.sum[v][2] = se[j];
    }
  }
  __syncthreads();
  if (per_depth && wave == 0 && lane < D) {
    float t = 0.0f, k = 0.0f, a = 0.0f;
    int32_t w = 0;
    for (int v = 0; v < kStatsVirtualWaves; ++v) {
      t += S.tested[v][lane];
      k += S.kept[v][lane];
      a += S.asum[v][lane];
      w += S.with[v][lane];
    }
    per_depth[lane] = t;
    per_depth[D + lane] = k;
    per_depth[2 * D + lane] = w ? a / (float)w : 0.0f;
  }
  if (summary && threadIdx.x == 0) {
    float t = 0.0f, n = 0.0f, e = 0.0f;
    for (int v = 0; v < kStatsVirtualWaves; ++v) {
      t += S.sum[v][0];
      n += S.sum[v][1];
      e += S.sum[v][2];
    }
    summary[0] = B ? 1.0f + t / (float)B : 0.0f;
    summary[1] = B ? 1.0f + e / (float)B : 0.0f;
    summary[2] = n > 0.0f ? t / n : 0.0f;
    summary[3] = n;
  }
}

}  // namespace sv
