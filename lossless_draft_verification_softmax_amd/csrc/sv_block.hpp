// sv_block.hpp -- workgroup-level reductions and the online-softmax group
// update shared by the row-pass and accept kernels.  Every reduction uses a
// fixed tree (DPP / permlane inside the wavefront, wavefront partials in
// order), so results are reproducible run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.hpp"

namespace sv {

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which makes every wave wait for all of its outstanding vector loads
// (the vmcnt counter is in order) and would drain the prefetched rows of the
// streaming loops at every reduction.  All intra-workgroup communication here
// goes through LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float block_sum_f(float v, float* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  lds_barrier();
  float t = 0.0f;
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += lds[w];
  lds_barrier();
  return t;
}

__device__ __forceinline__ double block_sum_d(double v, double* lds) {
  for (int m = 1; m < kWave; m <<= 1) v += shfl_xor_d(v, m);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  lds_barrier();
  double t = 0.0;
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += lds[w];
  lds_barrier();
  return t;
}

__device__ __forceinline__ SoftmaxPart block_merge(SoftmaxPart p, float sl, SoftmaxPart* lds) {
  p = wave_merge(p, sl);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = p;
  lds_barrier();
  SoftmaxPart t = lds[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) t = merge_parts(t, lds[w], sl);
  lds_barrier();
  return t;
}

// (value, index) arg max with NaN propagation and lowest index on ties.
struct ArgMax {
  float v;
  int32_t i;
};
__device__ __forceinline__ ArgMax argmax_merge(ArgMax a, ArgMax b) {
  if (a.v != a.v) return a;
  if (b.v != b.v) return b;
  if (a.v > b.v) return a;
  if (b.v > a.v) return b;
  return (a.i <= b.i) ? a : b;
}
__device__ __forceinline__ ArgMax block_argmax(ArgMax a, ArgMax* lds) {
  for (int m = 1; m < kWave; m <<= 1) {
    ArgMax o{__shfl_xor(a.v, m), __shfl_xor(a.i, m)};
    a = argmax_merge(a, o);
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = a;
  lds_barrier();
  ArgMax t = lds[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) t = argmax_merge(t, lds[w]);
  lds_barrier();
  return t;
}

// ---------------------------------------------------------------------------
// Row addressing.
template <typename E>
__device__ __forceinline__ const typename E::Storage* row_ptr(const void* base, int64_t row,
                                                             int64_t stride) {
  return static_cast<const typename E::Storage*>(base) + row * stride;
}

__device__ __forceinline__ bool temperature_ok(float T) { return T >= 0.0f && T < INFINITY; }

// ---------------------------------------------------------------------------
// Online softmax accumulation over one group of values (already widened).
// Masked (-inf) entries add nothing; a NaN or +inf poisons the state so that
// the row reads invalid.
template <int N>
__device__ __forceinline__ void softmax_group(SoftmaxPart& s, const float (&x)[N], float sl) {
  // products stay rounded products: no multiply is fused into a later add
  // (the fused multiply-adds below are explicit)
#pragma clang fp contract(off)
  float cm = x[0];
#pragma unroll
  for (int i = 1; i + 1 < N; i += 2) cm = vmax3(cm, x[i], x[i + 1]);
  if constexpr ((N % 2) == 0) cm = vmax(cm, x[N - 1]);
  const float mn = vmax(s.m, cm);
  const float ms = (mn == -INFINITY) ? 0.0f : mn;
  // The state's sum is relative to 2^R(s.m), R the integer reference: the
  // rescale 2^(R(s.m) - R(mn)) is exact, and 1 while the maximum holds.
  const float msl = ref_of(ms, sl);
  // exponentials in chunks of at most 8 (pairwise inside a chunk, chunks in
  // order), so that only 8 of them are live at a time
  constexpr int C = N < 8 ? N : 8;
  static_assert(N % C == 0, "group size must be a multiple of the chunk");
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < N; c += C) {
    float e[C];
#pragma unroll
    for (int i = 0; i < C; ++i) e[i] = exp2_fast(__builtin_fmaf(x[c + i], sl, -msl));
#pragma unroll
    for (int w = 1; w < C; w <<= 1) {
#pragma unroll
      for (int i = 0; i + w < C; i += 2 * w) e[i] += e[i + w];
    }
    acc = (c == 0) ? e[0] : acc + e[0];
  }
  const float scale = exp2_fast(ref_of(s.m, sl) - msl);
  s.z = __builtin_fmaf(s.z, scale, acc);
  s.m = mn;
}


}  // namespace sv
