// sv_confidence.hip -- the drafter's confidence in each drafted token, the
// input of the batch-shared budget ("AngelSpec: specialize the drafter...",
// section "D-cut": Figure 3 panel 1, the drafter emits confidence-scored
// candidates; equation A-hat multiplies the confidences along a request).
//
// conf[r][k] = q_k(d_k) = softmax(draft row k / T_r)[d_k], with T_r = 0 (a
// greedy drafter) scored at T = 1.  The draft rows are streamed once:
//   k_conf_part   one workgroup per (row, segment of 256 x 4 16-byte vectors):
//                 the segment's (max, sum 2^((x - max) sl)) into the
//                 workspace
//   k_conf_final  one thread per (r, k): the row's segment states merged in
//                 segment order, then 2^((x_d - max) sl) / sum.
// Both are HBM streams (the second reads a few bytes per row).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

constexpr int kConfThreads = 256;
constexpr int kConfVecs = 4;  // 16-byte vectors per thread per segment

template <typename E>
constexpr int64_t conf_segment() {
  return (int64_t)kConfThreads * kConfVecs * E::kPerVec;
}

int64_t confidence_segments(sv_dtype dtype, int64_t V) {
  const int64_t seg = (dtype == SV_DTYPE_BF16) ? conf_segment<Bf16>() : conf_segment<F32>();
  return (V + seg - 1) / seg;
}

// Scoring temperature of request r, or 0 when the request is invalid
// (negative, NaN or infinite temperature, depth outside [0, D]).
__device__ __forceinline__ float conf_sl(const ConfParams& c, int r, int* n) {
  *n = c.depth ? c.depth[r] : c.D;
  const float T = c.temperature[r];
  if (*n < 0 || *n > c.D || !temperature_ok(T)) return 0.0f;
  return kLog2e / (T > 0.0f ? T : 1.0f);
}

template <typename E>
__global__ __launch_bounds__(kConfThreads) void k_conf_part(ConfParams c) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  __shared__ SoftmaxPart lds[kConfThreads / kWave];
  const int64_t b = blockIdx.x;
  const int64_t row = b / c.nseg;  // r * D + k
  const int64_t seg = b % c.nseg;
  const int r = (int)(row / c.D), k = (int)(row % c.D);
  int n = 0;
  const float sl = conf_sl(c, r, &n);
  if (sl == 0.0f || k >= n) return;  // uniform: the final pass writes 0 or NaN
  const S* base = static_cast<const S*>(c.logits) + (c.row0[r] + k) * c.stride;
  const int64_t lo = seg * conf_segment<E>();
  const int64_t hi = min(c.V, lo + conf_segment<E>());
  float x[VEC * kConfVecs];
#pragma unroll
  for (int i = 0; i < kConfVecs; ++i) {
    const int64_t v0 = lo + ((int64_t)i * kConfThreads + threadIdx.x) * VEC;
    float* xi = &x[i * VEC];
    if (v0 + VEC <= hi) {
      E::unpack(load16(base + v0), xi);
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j) xi[j] = (v0 + j < hi) ? E::load1(base, v0 + j) : -INFINITY;
    }
  }
  SoftmaxPart s{-INFINITY, 0.0f};
  softmax_group<VEC * kConfVecs>(s, x, sl);
  s = block_merge(s, sl, lds);
  if (threadIdx.x == 0) c.part[row * c.nseg + seg] = make_float2(s.m, s.z);
}

template <typename E>
__global__ __launch_bounds__(kConfThreads) void k_conf_final(ConfParams c) {
  const int64_t idx = (int64_t)blockIdx.x * kConfThreads + threadIdx.x;
  if (idx >= (int64_t)c.B * c.D) return;
  const int r = (int)(idx / c.D), k = (int)(idx % c.D);
  int n = 0;
  const float sl = conf_sl(c, r, &n);
  if (sl == 0.0f) {
    c.conf[idx] = NAN;
    return;
  }
  if (k >= n) {
    c.conf[idx] = 0.0f;
    return;
  }
  SoftmaxPart s{-INFINITY, 0.0f};
  const float2* part = c.part + idx * c.nseg;
  for (int64_t j = 0; j < c.nseg; ++j) {
    const float2 v = part[j];
    s = merge_parts(s, SoftmaxPart{v.x, v.y}, sl);
  }
  const int32_t d = c.tokens[idx];
  const bool ok = s.m == s.m && fabsf(s.m) < INFINITY && d >= 0 && (int64_t)d < c.V;
  if (!ok) {
    c.conf[idx] = NAN;
    return;
  }
  const auto* base = static_cast<const typename E::Storage*>(c.logits) + (c.row0[r] + k) * c.stride;
  const float xd = E::load1(base, d);
  c.conf[idx] = exp2_fast((xd - s.m) * sl) / s.z;
}

template <typename E>
static hipError_t launch_conf_t(const ConfParams& c, hipStream_t stream) {
  const int64_t rows = (int64_t)c.B * c.D;
  hipLaunchKernelGGL(k_conf_part<E>, dim3((unsigned)(rows * c.nseg)), dim3(kConfThreads), 0, stream,
                     c);
  hipLaunchKernelGGL(k_conf_final<E>, dim3((unsigned)((rows + kConfThreads - 1) / kConfThreads)),
                     dim3(kConfThreads), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_confidence(const ConfParams& c, hipStream_t stream) {
  if ((int64_t)c.B * c.D == 0) return hipSuccess;
  return c.dtype == SV_DTYPE_BF16 ? launch_conf_t<Bf16>(c, stream) : launch_conf_t<F32>(c, stream);
}

}  // namespace sv
