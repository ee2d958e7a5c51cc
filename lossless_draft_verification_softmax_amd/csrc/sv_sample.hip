// sv_sample.hip -- one token per request drawn from softmax(row / T), on the
// verifier's Philox stream: the drafter side of the decode loop ([A] "MTP": a
// drafter proposes a block that the target then verifies in one pass;
// [T] "The MTP path": acceptance measured over whole generations).
//
// Request r draws from row row_base + row_index[r * index_stride] with the
// uniform u = (w2 >> 8) 2^-24, w2 the third word of the Philox4x32-10 block
// of counter (position, request_id, step, 0) -- words 0 and 1 of that block
// are the accept test's and the correction draw's at the same position.  The
// token is the smallest y whose cumulative weight exceeds u R, the weights
// being exp((x - max) / T) in float64 and R their total; at T = 0 it is the
// first arg max.  A row with a NaN or +inf entry or with every entry -inf, a
// negative row index and an invalid temperature give -1.
//
// One 1024-thread workgroup per request: thread t owns a contiguous chunk of
// the row; chunk sums in float64 are scanned in a fixed order (wavefront
// scan, then the wavefront totals in order); the thread whose chunk holds
// u R walks it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;

__device__ __forceinline__ double shfl_up_d(double v, int d) {
  int2 q = *reinterpret_cast<int2*>(&v);
  q.x = __shfl_up(q.x, d);
  q.y = __shfl_up(q.y, d);
  return *reinterpret_cast<double*>(&q);
}

template <typename E>
__global__ __launch_bounds__(kSampleThreads) void k_sample(SampleParams p) {
  using S = typename E::Storage;
  __shared__ float s_max[kSampleWaves];
  __shared__ int s_bad[kSampleWaves];
  __shared__ double s_tot[kSampleWaves];
  __shared__ int s_first[kSampleWaves];
  __shared__ int s_pick;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int32_t* out = p.tokens + (int64_t)r * p.token_stride;
  const int32_t ri = p.row_index[(int64_t)r * p.index_stride];
  const float T = p.temperature[r];
  if (ri < 0 || !temperature_ok(T)) {  // uniform
    if (tid == 0) *out = -1;
    return;
  }
  const S* row = static_cast<const S*>(p.logits) + (p.row_base + ri) * p.stride;
  const int64_t V = p.V;
  const int64_t chunk = (V + kSampleThreads - 1) / kSampleThreads;
  const int64_t lo = min(V, (int64_t)tid * chunk), hi = min(V, lo + chunk);

  // maximum (NaN and +inf mark the row invalid)
  float m = -INFINITY;
  int bad = 0;
  for (int64_t y = lo; y < hi; ++y) {
    const float x = E::load1(row, y);
    if (x != x || x == INFINITY) bad = 1;
    m = fmaxf(m, x);
  }
  m = wave_max(m);
  bad = __any(bad) ? 1 : 0;
  if (lane == 0) {
    s_max[wave] = m;
    s_bad[wave] = bad;
  }
  __syncthreads();
  m = s_max[0];
  bad = s_bad[0];
  for (int w = 1; w < kSampleWaves; ++w) {
    m = fmaxf(m, s_max[w]);
    bad |= s_bad[w];
  }
  if (bad || m == -INFINITY) {  // uniform
    if (tid == 0) *out = -1;
    return;
  }
  if (T == 0.0f) {
    // first index holding the maximum
    int first = INT32_MAX;
    for (int64_t y = lo; y < hi; ++y)
      if (E::load1(row, y) == m) {
        first = (int)y;
        break;
      }
    for (int o = 1; o < kWave; o <<= 1) first = min(first, __shfl_xor(first, o));
    if (lane == 0) s_first[wave] = first;
    __syncthreads();
    if (tid == 0) {
      int f = s_first[0];
      for (int w = 1; w < kSampleWaves; ++w) f = min(f, s_first[w]);
      *out = f;
    }
    return;
  }

  // float64 weights, chunk sums, fixed-order scan
  const double invT = 1.0 / (double)T;
  const double md = (double)m;
  double sum = 0.0;
  for (int64_t y = lo; y < hi; ++y) sum += exp(((double)E::load1(row, y) - md) * invT);
  double incl = sum;
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = shfl_up_d(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) s_tot[wave] = incl;
  __syncthreads();
  double base = 0.0, R = 0.0;
  for (int w = 0; w < kSampleWaves; ++w) {
    if (w < wave) base += s_tot[w];
    R += s_tot[w];
  }
  incl += base;
  const double excl = incl - sum;
  const Philox4 w4 = philox4x32_10(p.position, p.request_id ? p.request_id[r] : (uint32_t)r,
                                   p.step, 0u, p.seed_lo, p.seed_hi);
  const double t = (double)u24(w4.w[2]) * R;
  // the chunk holding t: the first with a positive sum whose inclusive value
  // exceeds t
  const bool holds = sum > 0.0 && incl > t;
  const uint64_t mask = __ballot(holds);
  if (lane == 0) s_first[wave] = mask ? (int)__builtin_ctzll(mask) : -1;
  if (tid == 0) s_pick = -1;
  __syncthreads();
  if (tid == 0) {
    for (int w = 0; w < kSampleWaves; ++w)
      if (s_first[w] >= 0) {
        s_pick = w * kWave + s_first[w];
        break;
      }
  }
  __syncthreads();
  const int pick = s_pick;
  if (pick >= 0) {
    if (tid == pick) {
      double c = excl;
      int y_out = -1;
      int last_pos = -1;
      for (int64_t y = lo; y < hi; ++y) {
        const double e = exp(((double)E::load1(row, y) - md) * invT);
        if (e > 0.0) last_pos = (int)y;
        c += e;
        if (e > 0.0 && c > t) {
          y_out = (int)y;
          break;
        }
      }
      // rounding left t at or past the chunk's running total: its last
      // token of positive weight
      *out = y_out >= 0 ? y_out : last_pos;
    }
    return;
  }
  // t at or past the total: the last token of positive weight
  int lastp = -1;
  for (int64_t y = hi - 1; y >= lo; --y)
    if (exp(((double)E::load1(row, y) - md) * invT) > 0.0) {
      lastp = (int)y;
      break;
    }
  for (int o = 1; o < kWave; o <<= 1) lastp = max(lastp, __shfl_xor(lastp, o));
  if (lane == 0) s_first[wave] = lastp;
  __syncthreads();
  if (tid == 0) {
    int f = -1;
    for (int w = 0; w < kSampleWaves; ++w) f = max(f, s_first[w]);
    *out = f;
  }
}

hipError_t launch_sample(const SampleParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  if (p.dtype == SV_DTYPE_BF16)
    hipLaunchKernelGGL(k_sample<Bf16>, dim3((unsigned)p.B), dim3(kSampleThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_sample<F32>, dim3((unsigned)p.B), dim3(kSampleThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
