// sv_confidence.hip -- the drafter's confidence in each drafted token, the
// input of the batch-shared budget ("AngelSpec: specialize the drafter...",
// section "D-cut": Figure 3 panel 1, the drafter emits confidence-scored
// candidates; equation A-hat multiplies the confidences along a request).
//
// conf[r][k] = q_k(d_k) = softmax(draft row k / T_r)[d_k], with T_r = 0 (a
// greedy drafter) scored at T = 1.  The draft rows are streamed once:
//   k_conf_part   persistent workgroups walk (row, segment) items, a segment
//                 being 256 x 8 whole 16-byte vectors of a row; the next
//                 item's loads are issued before the current one is reduced,
//                 and each wavefront writes its own (max, sum 2^((x - max)
//                 sl)) state, so the loop has no barrier
//   k_conf_final  one wavefront per (r, k): the row's wavefront states and
//                 its last partial vector (V mod 8 or V mod 4 elements)
//                 merged in a fixed order, then 2^((x_d - max) sl) / sum.
// The first is an HBM stream; the second reads a few bytes per row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

constexpr int kConfThreads = 256;
constexpr int kConfWaves = kConfThreads / kWave;
constexpr int kConfVecs = 8;     // 16-byte vectors per thread per segment
constexpr int kConfGrid = 1024;  // persistent workgroups (4 per CU: 110 VGPRs)

// Segments per row: whole vectors only; 0 when a row is shorter than one.
int64_t confidence_segments(sv_dtype dtype, int64_t V) {
  const int64_t vec = (dtype == SV_DTYPE_BF16) ? 8 : 4;
  const int64_t segv = (int64_t)kConfThreads * kConfVecs;
  return (V / vec + segv - 1) / segv;
}

int64_t confidence_states(sv_dtype dtype, int64_t V) {
  return confidence_segments(dtype, V) * kConfWaves;
}

// Scoring temperature of request r, or 0 when the request is invalid
// (negative, NaN or infinite temperature, depth outside [0, D]).
__device__ __forceinline__ float conf_sl(const ConfParams& c, int r, int* n) {
  *n = c.depth ? c.depth[r] : c.D;
  const float T = c.temperature[r];
  if (*n < 0 || *n > c.D || !temperature_ok(T)) return 0.0f;
  return kLog2e / (T > 0.0f ? T : 1.0f);
}

// -inf line read by lanes without data, so that every iteration issues the
// same loads (no data-dependent branch around them).
__device__ uint4 kConfNegInf[2] = {{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u},
                                   {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u}};

template <typename E>
struct ConfItem {
  int64_t row;  // r * D + k
  int64_t seg;
  float sl;     // 0: nothing to do for this item
};

template <typename E>
__device__ __forceinline__ ConfItem<E> conf_item(const ConfParams& c, int64_t b) {
  ConfItem<E> it;
  it.row = b / c.nseg;
  it.seg = b % c.nseg;
  const int r = (int)(it.row / c.D), k = (int)(it.row % c.D);
  int n = 0;
  it.sl = conf_sl(c, r, &n);
  if (k >= n) it.sl = 0.0f;
  return it;
}

template <typename E>
__device__ __forceinline__ void conf_load(const ConfParams& c, const ConfItem<E>& it,
                                          uint4 (&v)[kConfVecs]) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  const int r = (int)(it.row / c.D), k = (int)(it.row % c.D);
  const int64_t nvec = c.V / VEC;  // whole vectors of a row
  const S* base = static_cast<const S*>(c.logits) + (it.sl != 0.0f ? (c.row0[r] + k) * c.stride : 0);
  const uint4* dummy = &kConfNegInf[VEC == 8 ? 0 : 1];
#pragma unroll
  for (int i = 0; i < kConfVecs; ++i) {
    const int64_t q = (it.seg * kConfVecs + i) * kConfThreads + threadIdx.x;
    const bool in = it.sl != 0.0f && q < nvec;
    v[i] = load16(in ? (const void*)(base + q * VEC) : (const void*)dummy);
  }
}

template <typename E>
__global__ __launch_bounds__(kConfThreads) void k_conf_part(ConfParams c) {
  constexpr int VEC = E::kPerVec;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t items = (int64_t)c.B * c.D * c.nseg;
  int64_t b = blockIdx.x;
  if (b >= items) return;
  ConfItem<E> cur = conf_item<E>(c, b);
  uint4 v[kConfVecs];
  conf_load<E>(c, cur, v);
  for (; b < items; b += gridDim.x) {
    // issue the next item's loads, then reduce the current one
    const int64_t nb = b + gridDim.x;
    ConfItem<E> nxt = cur;
    uint4 w[kConfVecs];
    if (nb < items) {  // uniform
      nxt = conf_item<E>(c, nb);
      conf_load<E>(c, nxt, w);
    }
    if (cur.sl != 0.0f) {
      float x[VEC * kConfVecs];
#pragma unroll
      for (int i = 0; i < kConfVecs; ++i) E::unpack(v[i], &x[i * VEC]);
      SoftmaxPart s{-INFINITY, 0.0f};
      softmax_group<VEC * kConfVecs>(s, x, cur.sl);
      s = wave_merge(s, cur.sl);
      if (lane == 0)
        c.part[(cur.row * c.nseg + cur.seg) * kConfWaves + wave] = make_float2(s.m, s.z);
    }
    cur = nxt;
#pragma unroll
    for (int i = 0; i < kConfVecs; ++i) v[i] = w[i];
  }
}

// One wavefront per (r, k): lane l merges states l, l + 64, ... in order and
// the row's last partial vector (element nvec * VEC + l, l < V mod VEC),
// then the wavefront's states are merged by the fixed tree of wave_merge.
template <typename E>
__global__ __launch_bounds__(kConfThreads) void k_conf_final(ConfParams c) {
  constexpr int VEC = E::kPerVec;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t idx = (int64_t)blockIdx.x * kConfWaves + threadIdx.x / kWave;
  if (idx >= (int64_t)c.B * c.D) return;  // uniform per wavefront
  const int r = (int)(idx / c.D), k = (int)(idx % c.D);
  int n = 0;
  const float sl = conf_sl(c, r, &n);
  if (sl == 0.0f || k >= n) {
    if (lane == 0) c.conf[idx] = (sl == 0.0f) ? NAN : 0.0f;
    return;
  }
  const auto* base = static_cast<const typename E::Storage*>(c.logits) + (c.row0[r] + k) * c.stride;
  SoftmaxPart s{-INFINITY, 0.0f};
  const int64_t nstate = c.nseg * kConfWaves;
  const float2* part = c.part + idx * nstate;
  for (int64_t j = lane; j < nstate; j += kWave) {
    const float2 v = part[j];
    s = merge_parts(s, SoftmaxPart{v.x, v.y}, sl);
  }
  const int64_t tail = (c.V / VEC) * VEC + lane;
  if (tail < c.V) {
    float x1[1] = {E::load1(base, tail)};
    softmax_group<1>(s, x1, sl);
  }
  s = wave_merge(s, sl);
  if (lane != 0) return;
  const int32_t d = c.tokens[idx];
  const bool ok = s.m == s.m && fabsf(s.m) < INFINITY && d >= 0 && (int64_t)d < c.V;
  if (!ok) {
    c.conf[idx] = NAN;
    return;
  }
  const float xd = E::load1(base, d);
  c.conf[idx] = exp2_fast(__builtin_fmaf(xd, sl, -ref_of(s.m, sl))) / s.z;
}

template <typename E>
static hipError_t launch_conf_t(const ConfParams& c, hipStream_t stream) {
  const int64_t rows = (int64_t)c.B * c.D;
  const int64_t items = rows * c.nseg;
  if (items > 0) {
    const unsigned grid = (unsigned)(items < kConfGrid ? items : kConfGrid);
    hipLaunchKernelGGL(k_conf_part<E>, dim3(grid), dim3(kConfThreads), 0, stream, c);
  }
  hipLaunchKernelGGL(k_conf_final<E>, dim3((unsigned)((rows + kConfWaves - 1) / kConfWaves)),
                     dim3(kConfThreads), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_confidence(const ConfParams& c, hipStream_t stream) {
  if ((int64_t)c.B * c.D == 0) return hipSuccess;
  return c.dtype == SV_DTYPE_BF16 ? launch_conf_t<Bf16>(c, stream) : launch_conf_t<F32>(c, stream);
}

}  // namespace sv
