// sv_rowpass.hip -- the HBM-streaming statistics pass of verification.
//
// For every verified position the target scores the drafted token in one
// pass over the vocabulary ("Tencent open-sources AngelSpec", section "Why one
// universal drafter underperforms"); per row this needs the softmax
// normaliser (max and sum of 2^((x - max) log2(e) / T)) and, for the
// acceptance rate of equation L_e2e ("AngelSpec: specialize the drafter...",
// section "MTP"), sum_y min(p(y), q(y)) over the target / draft row pair.
//
//   k_plan     one workgroup: scans depth / temperature and writes the work
//              list: every (request, position) row pair at T > 0, then every
//              single row (bonus rows at T > 0, all target rows at T = 0).
//   k_rowpass  persistent, one 1024-thread workgroup per CU, items taken
//              round-robin.  A row pair is one item: pass 1 streams both rows
//              from HBM with 16-byte loads (online max / sum), then pass 2
//              streams them again for sum min(p, q).  At most one row pair
//              per CU is in flight (about 155 MB on 256 CUs), so pass 2 reads
//              what pass 1 just pulled into the 256 MB Infinity Cache.  Single
//              rows are cut into segments (one pass each) and fill the tail.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

constexpr int kPassThreads = 1024;
constexpr int kPassUnroll = 4;
constexpr int kPlanThreads = 1024;

// ---------------------------------------------------------------------------
// Exclusive prefix sums of two ints over the block (fixed order, one pair of
// barriers for both); tot gets the block totals.
__device__ __forceinline__ int2 block_excl_scan_i2(int2 v, int2* lds, int2* tot) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int2 x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int ox = __shfl_up(x.x, d), oy = __shfl_up(x.y, d);
    if (lane >= d) {
      x.x += ox;
      x.y += oy;
    }
  }
  if (lane == kWave - 1) lds[wave] = x;
  lds_barrier();
  int2 base = make_int2(0, 0), t = make_int2(0, 0);
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
    const int2 o = lds[w];
    if (w < wave) {
      base.x += o.x;
      base.y += o.y;
    }
    t.x += o.x;
    t.y += o.y;
  }
  lds_barrier();
  *tot = t;
  return make_int2(base.x + x.x - v.x, base.y + x.y - v.y);
}

__global__ __launch_bounds__(kPlanThreads) void k_plan(VerifyParams p) {
  __shared__ int2 lds[kPlanThreads / kWave];
  int32_t carry_pairs = 0, carry_singles = 0;
  for (int base = 0; base < p.B; base += kPlanThreads) {
    const int r = base + (int)threadIdx.x;
    int32_t np = 0, ns = 0, n = 0;
    float T = 0.0f;
    int64_t t0 = 0, d0 = 0;
    if (r < p.B) {
      p.fb_done[r] = 0;
      // every load of the request at once
      n = p.depth[r];
      T = p.temperature[r];
      t0 = p.target_row0[r];
      if (p.draft_row0) d0 = p.draft_row0[r];
      const bool valid = n >= 0 && n <= p.D && temperature_ok(T) &&
                         !(T > 0.0f && n > 0 && p.draft == nullptr);
      if (valid) {
        np = (T > 0.0f) ? n : 0;
        ns = (T > 0.0f) ? 1 : n + 1;
      }
    }
    int2 tot;
    const int2 off = block_excl_scan_i2(make_int2(np, ns), lds, &tot);
    const int32_t op = carry_pairs + off.x;
    const int32_t os = carry_singles + off.y;
    if (np > 0 || ns > 0) {
      const float sl = (T > 0.0f) ? kLog2e / T : 0.0f;
      for (int k = 0; k < np; ++k)
        p.plan_pairs[op + k] = PlanItem{t0 + k, d0 + k, ((uint32_t)r << 7) | (uint32_t)k, T, sl, 0u};
      for (int j = 0; j < ns; ++j) {
        const int k = (T > 0.0f) ? n : j;
        p.plan_singles[os + j] = PlanItem{t0 + k, 0, ((uint32_t)r << 7) | (uint32_t)k, T, sl, 0u};
      }
    }
    carry_pairs += tot.x;
    carry_singles += tot.y;
  }
  if (threadIdx.x == 0) {
    p.plan_counts[0] = carry_pairs;
    p.plan_counts[1] = carry_singles;
    *p.sync_error = 0;
    *p.fb_count = 0;  // float64 draw queue, appended to by k_accept_draw
  }
  if (p.nshard > 1 && threadIdx.x < 2 * kMaxShards) {
    const int s = (int)threadIdx.x % kMaxShards;
    p.shard_tab[threadIdx.x] = (int)threadIdx.x < kMaxShards ? p.tsh[s] : p.dsh[s];
  }
  // The team row pass tells fresh exchange words from stale ones by their tag
  // (never 0 once written): clear the words this launch reads (4 records of
  // 4 words per team member) before every launch.
  const int64_t used = p.team > 0 ? (int64_t)p.nteams * p.team * 16 : 0;
  uint4* xch = reinterpret_cast<uint4*>(p.team_xch);
  for (int64_t i = threadIdx.x; i < used / 2; i += kPlanThreads) xch[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// Streaming loops.  A thread's share of [lo, hi) is the vectors
// lo + VEC * (tid + j * blockDim); they are taken in batches of kPassUnroll
// vectors per row, and the loads of the next batch are issued before the
// current batch is processed (two register buffers), so every wave keeps
// loads in flight while it computes.

template <typename E, bool kPair>
struct Batch {
  uint4 p[kPassUnroll];
  uint4 q[kPair ? kPassUnroll : 1];
};

template <typename E, bool kPair>
__device__ __forceinline__ void load_batch(Batch<E, kPair>& b, const typename E::Storage* prow,
                                           const typename E::Storage* qrow, int64_t base,
                                           int64_t step, int64_t vhi) {
  const uint4 pad = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
#pragma unroll
  for (int u = 0; u < kPassUnroll; ++u) {
    const int64_t i = base + u * step;
    b.p[u] = (i < vhi) ? load16_keep(prow + i) : pad;
    if constexpr (kPair) b.q[u] = (i < vhi) ? load16_keep(qrow + i) : pad;
  }
}

template <typename E, bool kPair>
__device__ __forceinline__ void softmax_batch(const Batch<E, kPair>& b, float sl, SoftmaxPart& sp,
                                              SoftmaxPart& sq) {
  constexpr int VEC = E::kPerVec;
  constexpr int G = VEC * kPassUnroll;
  float x[G];
#pragma unroll
  for (int u = 0; u < kPassUnroll; ++u)
    E::unpack(b.p[u], *reinterpret_cast<float(*)[VEC]>(&x[u * VEC]));
  softmax_group<G>(sp, x, sl);
  if constexpr (kPair) {
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u)
      E::unpack(b.q[u], *reinterpret_cast<float(*)[VEC]>(&x[u * VEC]));
    softmax_group<G>(sq, x, sl);
  }
}

// Pass 1 over [lo, hi) of one row (and its partner row when kPair).
template <typename E, bool kPair>
__device__ __forceinline__ void stream_softmax(const typename E::Storage* prow,
                                               const typename E::Storage* qrow, int64_t lo,
                                               int64_t hi, float sl, SoftmaxPart& sp,
                                               SoftmaxPart& sq) {
  constexpr int VEC = E::kPerVec;
  const int64_t vhi = lo + ((hi - lo) / VEC) * VEC;
  const int64_t step = (int64_t)blockDim.x * VEC;
  const int64_t batch = step * kPassUnroll;
  int64_t base = lo + (int64_t)threadIdx.x * VEC;
  Batch<E, kPair> b0, b1;
  if (base < vhi) load_batch<E, kPair>(b0, prow, qrow, base, step, vhi);
  for (; base < vhi; base += 2 * batch) {
    if (base + batch < vhi) load_batch<E, kPair>(b1, prow, qrow, base + batch, step, vhi);
    softmax_batch<E, kPair>(b0, sl, sp, sq);
    if (base + batch >= vhi) break;
    if (base + 2 * batch < vhi) load_batch<E, kPair>(b0, prow, qrow, base + 2 * batch, step, vhi);
    softmax_batch<E, kPair>(b1, sl, sp, sq);
  }
  for (int64_t i = vhi + threadIdx.x; i < hi; i += blockDim.x) {
    float x1[1] = {E::load1(prow, i)};
    softmax_group<1>(sp, x1, sl);
    if constexpr (kPair) {
      x1[0] = E::load1(qrow, i);
      softmax_group<1>(sq, x1, sl);
    }
  }
}

template <typename E>
__device__ __forceinline__ float overlap_batch(const Batch<E, true>& b, float sl, float cp,
                                               float cq, float dlz) {
  constexpr int VEC = E::kPerVec;
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kPassUnroll; ++u) {
    float a[VEC], c[VEC], e[VEC];
    E::unpack(b.p[u], a);
    E::unpack(b.q[u], c);
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      e[j] = exp2_fast(fminf(__builtin_fmaf(a[j], sl, -cp), __builtin_fmaf(c[j], sl, -cq) - dlz));
#pragma unroll
    for (int w = 1; w < VEC; w <<= 1) {
#pragma unroll
      for (int j = 0; j + w < VEC; j += 2 * w) e[j] += e[j + w];
    }
    acc += e[0];
  }
  return acc;
}

// Pass 2: this thread's share of sum_y 2^min(x_p(y) sl - cp, x_q(y) sl - cq - dlz)
// with the rows' references cp = R(m_p), cq = R(m_q) and dlz = lz_q -
// lz_p, the difference of the log2 sums against them: 2^lz_p times the sum
// of min(p, q) (padding vectors are -inf and add 0).
template <typename E>
__device__ __forceinline__ float stream_overlap(const typename E::Storage* prow,
                                                const typename E::Storage* qrow, int64_t V,
                                                float sl, float cp, float cq, float dlz) {
  constexpr int VEC = E::kPerVec;
  const int64_t vhi = (V / VEC) * VEC;
  const int64_t step = (int64_t)blockDim.x * VEC;
  const int64_t batch = step * kPassUnroll;
  int64_t base = (int64_t)threadIdx.x * VEC;
  float acc = 0.0f;
  Batch<E, true> b0, b1;
  if (base < vhi) load_batch<E, true>(b0, prow, qrow, base, step, vhi);
  for (; base < vhi; base += 2 * batch) {
    if (base + batch < vhi) load_batch<E, true>(b1, prow, qrow, base + batch, step, vhi);
    acc += overlap_batch<E>(b0, sl, cp, cq, dlz);
    if (base + batch >= vhi) break;
    if (base + 2 * batch < vhi) load_batch<E, true>(b0, prow, qrow, base + 2 * batch, step, vhi);
    acc += overlap_batch<E>(b1, sl, cp, cq, dlz);
  }
  for (int64_t i = vhi + threadIdx.x; i < V; i += blockDim.x) {
    const float a = E::load1(prow, i), c = E::load1(qrow, i);
    acc += exp2_fast(fminf(__builtin_fmaf(a, sl, -cp), __builtin_fmaf(c, sl, -cq) - dlz));
  }
  return acc;
}

template <typename E>
__device__ void pair_item(const VerifyParams& p, const PlanItem& it, SoftmaxPart* lds_sm,
                          float* lds_f) {
  const int r = (int)(it.code >> 7), k = (int)(it.code & 127u);
  const float sl = kLog2e / it.T;
  const auto* prow = row_ptr<E>(p.target, it.trow, p.stride);
  const auto* qrow = row_ptr<E>(p.draft, it.drow, p.stride);
  SoftmaxPart sp{-INFINITY, 0.0f}, sq{-INFINITY, 0.0f};
  stream_softmax<E, true>(prow, qrow, 0, p.V, sl, sp, sq);
  sp = block_merge(sp, sl, lds_sm);
  sq = block_merge(sq, sl, lds_sm);
  const int64_t unit = (int64_t)r * (p.D + 1) + k;
  const int64_t slot = unit * p.S1;
  if (threadIdx.x == 0) {
    // the row states, and the same as the one slice state of the pair
    p.pair_p[unit] = make_float2(sp.m, sp.z);
    p.pair_q[unit] = make_float2(sq.m, sq.z);
    p.part_p[slot] = make_float2(sp.m, sp.z);
    p.part_q[slot] = make_float2(sq.m, sq.z);
  }
  float a = 0.0f;
  const bool finite = sp.m == sp.m && sq.m == sq.m && fabsf(sp.m) < INFINITY &&
                      fabsf(sq.m) < INFINITY;
  if (finite) {  // block-uniform
    const float lzp = __log2f(sp.z);
    const float dlz = __log2f(sq.z) - lzp;
    a = block_sum_f(stream_overlap<E>(prow, qrow, p.V, sl, ref_of(sp.m, sl), ref_of(sq.m, sl),
                                      dlz),
                    lds_f) *
        exp2_fast(-lzp);
  }
  if (threadIdx.x == 0) p.part_a[slot] = a;
}

template <typename E>
__device__ void single_item(const VerifyParams& p, const PlanItem& it, int seg,
                            SoftmaxPart* lds_sm, ArgMax* lds_am) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  const int r = (int)(it.code >> 7), k = (int)(it.code & 127u);
  const float T = it.T;
  const S* prow = row_ptr<E>(p.target, it.trow, p.stride);
  const int64_t lo = (int64_t)seg * p.seg1;
  const int64_t hi = min(p.V, lo + (int64_t)p.seg1);
  const int64_t slot = ((int64_t)r * (p.D + 1) + k) * p.S1 + seg;
  if (T > 0.0f) {
    const float sl = kLog2e / T;
    SoftmaxPart sp{-INFINITY, 0.0f}, unused{-INFINITY, 0.0f};
    if (hi > lo) stream_softmax<E, false>(prow, nullptr, lo, hi, sl, sp, unused);
    sp = block_merge(sp, sl, lds_sm);
    if (threadIdx.x == 0) p.part_p[slot] = make_float2(sp.m, sp.z);
    return;
  }
  // T = 0: arg max over the segment.  Per thread the best vector (strictly
  // greater keeps the earliest; NaN propagates through the maximum), then the
  // first maximal element inside it.
  const int64_t vhi = (hi > lo) ? lo + ((hi - lo) / VEC) * VEC : lo;
  const int64_t step = (int64_t)blockDim.x * VEC;
  float best = -INFINITY;
  int64_t bvec = -1;
  const int64_t batch = step * kPassUnroll;
  auto argmax_batch = [&](const Batch<E, false>& bt, int64_t b0) {
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      float x[VEC];
      E::unpack(bt.p[u], x);
      float cm = x[0];
#pragma unroll
      for (int j = 1; j < VEC; ++j) cm = vmax(cm, x[j]);
      const bool up = cm > best;
      best = vmax(best, cm);
      bvec = up ? b0 + u * step : bvec;
    }
  };
  int64_t base = lo + (int64_t)threadIdx.x * VEC;
  Batch<E, false> b0, b1;
  if (base < vhi) load_batch<E, false>(b0, prow, nullptr, base, step, vhi);
  for (; base < vhi; base += 2 * batch) {
    if (base + batch < vhi) load_batch<E, false>(b1, prow, nullptr, base + batch, step, vhi);
    argmax_batch(b0, base);
    if (base + batch >= vhi) break;
    if (base + 2 * batch < vhi) load_batch<E, false>(b0, prow, nullptr, base + 2 * batch, step, vhi);
    argmax_batch(b1, base + batch);
  }
  ArgMax a{best, INT32_MAX};
  if (best == best && bvec >= 0) {
    float x[VEC];
    E::unpack(load16_keep(prow + bvec), x);
#pragma unroll
    for (int j = VEC - 1; j >= 0; --j)
      if (x[j] == best) a.i = (int32_t)(bvec + j);
  }
  for (int64_t i = vhi + threadIdx.x; i < hi; i += blockDim.x)
    a = argmax_merge(a, ArgMax{E::load1(prow, i), (int32_t)i});
  a = block_argmax(a, lds_am);
  if (threadIdx.x == 0) p.part_p[slot] = make_float2(a.v, __int_as_float(a.i));
}

template <typename E>
__global__ __launch_bounds__(kPassThreads) void k_rowpass(VerifyParams p) {
  __shared__ SoftmaxPart lds_sm[kPassThreads / kWave];
  __shared__ ArgMax lds_am[kPassThreads / kWave];
  __shared__ float lds_f[kPassThreads / kWave];
  const int64_t n_pairs = p.plan_counts[0];
  const int64_t n_singles = p.plan_counts[1];
  const int64_t total = n_pairs + n_singles * p.S1;
  for (int64_t it = blockIdx.x; it < total; it += gridDim.x) {
    if (it < n_pairs) {
      pair_item<E>(p, p.plan_pairs[it], lds_sm, lds_f);
    } else {
      const int64_t j = it - n_pairs;
      single_item<E>(p, p.plan_singles[j / p.S1], (int)(j % p.S1), lds_sm, lds_am);
    }
  }
}

void launch_plan(const VerifyParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, stream, p);
}

void launch_rowpass(const VerifyParams& p, int grid, hipStream_t stream) {
  if (p.dtype == SV_DTYPE_BF16)
    hipLaunchKernelGGL(k_rowpass<Bf16>, dim3((unsigned)grid), dim3(kPassThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_rowpass<F32>, dim3((unsigned)grid), dim3(kPassThreads), 0, stream, p);
}

}  // namespace sv
