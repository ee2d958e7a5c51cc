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
// being exp((x - max) / T) and R their total; at T = 0 it is the first arg
// max.  A row with a NaN or +inf entry or with every entry -inf, a negative
// row index and an invalid temperature give -1.
//
// One 1024-thread workgroup per request.  Thread t owns the contiguous chunk
// [t c, (t + 1) c) of the row, c = ceil(V / 1024) rounded up to whole groups
// of 8 elements, read group by group (16-byte vector loads when the row is
// 16-byte aligned, else element by element; up to 64 bf16 or 32 fp32
// elements per thread stay in registers for every pass).  The weights are
// float64 exp((x - m) / T) (x - m taken in float64; the table-driven exp of
// the float64 draw, about 2 ulp), which holds at any temperature, each group summed as a tree, a thread's groups in order, then one
// fixed-order block scan of the thread sums (wavefront scans, then the
// wavefront totals in order); t = u R, and the thread whose chunk holds t
// walks it group by group and then inside the group.  A float32 pass would
// be cheaper per element, but its error bound (a few 1e-6 of R) puts about
// one draw in ten of these rows within reach of a boundary, so nearly every
// call of 64 requests would wait for a float64 recompute.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_drawrow.hpp"
#include "sv_exp64.hpp"
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

// Eight elements from i0 of a row (entries at or past hi read as -inf).
template <typename E>
__device__ __forceinline__ void group8(const typename E::Storage* row, bool aligned, int64_t i0,
                                       int64_t hi, float (&x)[kPer]) {
  if (aligned && i0 + kPer <= hi) {
    constexpr int NV = kPer / E::kPerVec;
    uint4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load16(row + i0 + k * E::kPerVec);
#pragma unroll
    for (int k = 0; k < NV; ++k) E::unpack(v[k], x + k * E::kPerVec);
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) x[j] = (i0 + j < hi) ? E::load1(row, i0 + j) : -INFINITY;
  }
}

// Group sum as a tree (((0+1)+(2+3))+((4+5)+(6+7))).
template <typename T>
__device__ __forceinline__ T tree8(const T (&w)[kPer]) {
  return ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
}

// Block inclusive scan of one value per thread in a fixed order; *total gets
// the block total.  LDS: kSampleWaves values.
template <typename T>
__device__ __forceinline__ T block_scan(T v, T* lds, T* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T o;
    if constexpr (sizeof(T) == 8) o = shfl_up_d(v, d);
    else o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == kWave - 1) lds[wave] = v;
  __syncthreads();
  T base = T(0), tot = T(0);
  for (int w = 0; w < kSampleWaves; ++w) {
    if (w < wave) base += lds[w];
    tot += lds[w];
  }
  __syncthreads();
  *total = tot;
  return base + v;
}

// The first thread (in order) whose flag is set, or -1.  LDS: kSampleWaves.
__device__ __forceinline__ int block_first(bool flag, int* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint64_t mask = __ballot(flag);
  if (lane == 0) lds[wave] = mask ? (int)__builtin_ctzll(mask) : -1;
  __syncthreads();
  int first = -1;
  for (int w = 0; w < kSampleWaves; ++w)
    if (lds[w] >= 0) {
      first = w * kWave + lds[w];
      break;
    }
  __syncthreads();
  return first;
}

// Elements per thread: ceil(V / 1024) rounded up to whole groups of 8.
__device__ __forceinline__ int64_t sample_chunk(int64_t V) {
  return ((V + kSampleThreads - 1) / kSampleThreads + kPer - 1) / kPer * kPer;
}

struct SampleLds {
  double tab[kExp64Table];  // 2^(j/256) for exp64_tab
  float f[kSampleWaves];
  double d[kSampleWaves];
  int i[kSampleWaves];
  int pick;
};

// A thread's chunk, group by group: held in registers (NC > 0: the row is
// 16-byte aligned and the chunk at most NC whole groups; every load is issued
// at once and each pass reads the registers) or read from memory at each
// pass (NC = 0).  each(f) calls f(g, x) for the chunk's groups in order, x
// the group's eight values (-inf past the row's end); f returns false to
// stop.
template <typename E, int NC>
struct Chunk {
  static constexpr int NV = kPer / E::kPerVec;
  const typename E::Storage* row;
  bool aligned;
  int64_t lo, hi;
  uint4 v[NC > 0 ? NC * NV : 1];
  __device__ __forceinline__ void load() {
    if constexpr (NC > 0) {
#pragma unroll
      for (int g = 0; g < NC; ++g)
        if (lo + (int64_t)(g + 1) * kPer <= hi) {
#pragma unroll
          for (int k = 0; k < NV; ++k) v[g * NV + k] = load16(row + lo + g * kPer + k * E::kPerVec);
        }
    }
  }
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
    if constexpr (NC > 0) {
      bool go = true;
#pragma unroll
      for (int g = 0; g < NC; ++g) {
        const int64_t i0 = lo + (int64_t)g * kPer;
        if (go && i0 < hi) {
          float x[kPer];
          if (i0 + kPer <= hi) {
#pragma unroll
            for (int k = 0; k < NV; ++k) E::unpack(v[g * NV + k], x + k * E::kPerVec);
          } else {  // the row's ragged end
#pragma unroll
            for (int j = 0; j < kPer; ++j) x[j] = (i0 + j < hi) ? E::load1(row, i0 + j) : -INFINITY;
          }
          go = f(i0, x);
        }
      }
    } else {
      for (int64_t i0 = lo; i0 < hi; i0 += kPer) {
        float x[kPer];
        group8<E>(row, aligned, i0, hi, x);
        if (!f(i0, x)) break;
      }
    }
  }
};

template <typename E, int NC>
__device__ __forceinline__ void sample_row(const SampleParams& p, int32_t* out, float T, float u,
                                           Chunk<E, NC>& ch, SampleLds& L) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  ch.load();
  // maximum (NaN and +inf mark the row invalid)
  float m = -INFINITY;
  int bad = 0;
  ch.each([&](int64_t, const float (&x)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (x[j] != x[j] || x[j] == INFINITY) bad = 1;
      m = fmaxf(m, x[j]);
    }
    return true;
  });
  m = wave_max(m);
  bad = __any(bad) ? 1 : 0;
  if (lane == 0) {
    L.f[wave] = m;
    L.i[wave] = bad;
  }
  __syncthreads();
  m = L.f[0];
  bad = L.i[0];
  for (int w = 1; w < kSampleWaves; ++w) {
    m = fmaxf(m, L.f[w]);
    bad |= L.i[w];
  }
  __syncthreads();
  if (bad || m == -INFINITY) {  // uniform
    if (tid == 0) *out = -1;
    return;
  }
  if (T == 0.0f) {
    // first index holding the maximum
    int first = INT32_MAX;
    ch.each([&](int64_t i0, const float (&x)[kPer]) {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (first == INT32_MAX && x[j] == m) first = (int)(i0 + j);
      return first == INT32_MAX;
    });
    for (int o = 1; o < kWave; o <<= 1) first = min(first, __shfl_xor(first, o));
    if (lane == 0) L.i[wave] = first;
    __syncthreads();
    if (tid == 0) {
      int f = L.i[0];
      for (int w = 1; w < kSampleWaves; ++w) f = min(f, L.i[w]);
      *out = f;
    }
    return;
  }

  // ---- float64 weights exp((x - m) / T), group sums as a tree ----
  const double invT = 1.0 / (double)T;
  const double md = (double)m;
  double sum = 0.0;
  ch.each([&](int64_t, const float (&x)[kPer]) {
    double w[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) w[j] = exp64_tab(((double)x[j] - md) * invT, L.tab);
    sum += tree8(w);
    return true;
  });
  double R;
  const double incl = block_scan<double>(sum, L.d, &R);
  const double excl = incl - sum;
  const double t = (double)u * R;
  // the chunk holding t: the first with a positive sum whose inclusive value
  // exceeds t
  const int pick = block_first(sum > 0.0 && incl > t, L.i);
  if (pick >= 0) {
    if (tid == pick) {
      double c = excl;
      int y_out = -1;
      int last_pos = -1;
      ch.each([&](int64_t i0, const float (&x)[kPer]) {
        double w[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) w[j] = exp64_tab(((double)x[j] - md) * invT, L.tab);
        const double gs = tree8(w);
        if (!(c + gs > t)) {  // the whole group lies below t
          c += gs;
#pragma unroll
          for (int j = 0; j < kPer; ++j)
            if (w[j] > 0.0) last_pos = (int)(i0 + j);
          return true;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          if (y_out < 0) {
            if (w[j] > 0.0) last_pos = (int)(i0 + j);
            c += w[j];
            if (w[j] > 0.0 && c > t) y_out = (int)(i0 + j);
          }
        }
        return y_out < 0;
      });
      // rounding left t at or past the chunk's running total: its last
      // token of positive weight
      *out = y_out >= 0 ? y_out : last_pos;
    }
    return;
  }
  // t at or past the total: the last token of positive weight
  int lastp = -1;
  ch.each([&](int64_t i0, const float (&x)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (exp64_tab(((double)x[j] - md) * invT, L.tab) > 0.0) lastp = (int)(i0 + j);
    return true;
  });
  for (int o = 1; o < kWave; o <<= 1) lastp = max(lastp, __shfl_xor(lastp, o));
  if (lane == 0) L.i[wave] = lastp;
  __syncthreads();
  if (tid == 0) {
    int f = -1;
    for (int w = 0; w < kSampleWaves; ++w) f = max(f, L.i[w]);
    *out = f;
  }
}

// Groups of a chunk held in registers: 8 (64 bf16 elements, 32 registers) or
// 4 (32 fp32 elements).
template <typename E>
constexpr int kSampleCached = E::kPerVec == 8 ? 8 : 4;

template <typename E>
__global__ __launch_bounds__(kSampleThreads) void k_sample(SampleParams p) {
  using S = typename E::Storage;
  __shared__ SampleLds L;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* out = p.tokens + (int64_t)r * p.token_stride;
  const int32_t ri = p.row_index[(int64_t)r * p.index_stride];
  const float T = p.temperature[r];
  if (ri < 0 || !temperature_ok(T)) {  // uniform
    if (tid == 0) *out = -1;
    return;
  }
  const S* row = static_cast<const S*>(p.logits) + (p.row_base + ri) * p.stride;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const int64_t V = p.V;
  const int64_t chunk = sample_chunk(V);
  const int64_t lo = min(V, (int64_t)tid * chunk), hi = min(V, lo + chunk);
  const Philox4 w4 = philox4x32_10(p.position, p.request_id ? p.request_id[r] : (uint32_t)r,
                                   p.step, 0u, p.seed_lo, p.seed_hi);
  const float u = u24(w4.w[2]);
  for (int j = tid; j < kExp64Table; j += kSampleThreads) L.tab[j] = kExp2Frac[j];
  // (the first barrier of sample_row orders these writes before any read)
  constexpr int NC = kSampleCached<E>;
  if (aligned && chunk <= NC * kPer) {  // uniform
    Chunk<E, NC> ch{row, aligned, lo, hi};
    sample_row<E, NC>(p, out, T, u, ch, L);
  } else {
    Chunk<E, 0> ch{row, aligned, lo, hi};
    sample_row<E, 0>(p, out, T, u, ch, L);
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
