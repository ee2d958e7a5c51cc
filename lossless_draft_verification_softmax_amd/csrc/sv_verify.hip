// sv_verify.hip -- batched lossless draft verification on gfx950.
//
// Method (the AngelSpec pages): the target scores every drafted position in
// one pass and verification is lossless rejection sampling
// ("Tencent open-sources AngelSpec", section "Why one universal drafter
// underperforms"); one rejection invalidates every later position
// ("AngelSpec: specialize the drafter...", section "MTP", after equation
// L_e2e); at T = 0 the test is an arg-max match ("The MTP path").
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   k_rowstats   per (request, position) row and vocabulary segment: online
//                softmax state (max, sum of 2^((x - max) sl)) of the target
//                row and the draft row, or (max, first arg max) at T = 0.
//                This is the HBM-streaming pass (16-byte loads).
//   k_alpha      same rows again: sum_y min(p, q) per segment (optional).
//   k_accept     one workgroup per request: merge the segments, Philox accept
//                test per position, wavefront ballot + first set bit = tau,
//                emitted drafts, alpha, the draw's normalisers.
//   k_draw_*     inverse-CDF draw of the correction / bonus token: float32
//                segment masses, then an LDS-staged block scan inside the
//                chosen segment; draws whose float32 CDF margin is under
//                1e-5 are recomputed in float64 by the same three steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

constexpr int kStatThreads = 256;
constexpr int kStatUnroll = 4;
constexpr int kDrawThreads = 256;
constexpr int kDrawPerThread = 8;
constexpr int kDrawTile = kDrawThreads * kDrawPerThread;
constexpr float kDrawMargin32 = 1e-5f;

// ---------------------------------------------------------------------------
// Block-level helpers.

// Inclusive prefix sum over the 256 threads of a block, in a fixed order
// (Hillis-Steele inside each wavefront, then the wave totals), so that two
// kernels scanning the same values get bit-identical results.  Returns the
// inclusive value; *total receives the block total (the last thread's value).
template <typename T>
__device__ __forceinline__ T block_inclusive_scan(T v, T* lds4, T* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T o;
    if constexpr (sizeof(T) == 8) {
      int2 p = *reinterpret_cast<int2*>(&v);
      p.x = __shfl_up(p.x, d);
      p.y = __shfl_up(p.y, d);
      o = *reinterpret_cast<T*>(&p);
    } else {
      o = __shfl_up(v, d);
    }
    if (lane >= d) v = v + o;
  }
  if (lane == kWave - 1) lds4[wave] = v;
  __syncthreads();
  T base = T(0);
  for (int w = 0; w < wave; ++w) base = base + lds4[w];
  T out = (wave == 0) ? v : base + v;
  T tot = lds4[0];
  for (int w = 1; w < kDrawThreads / kWave; ++w) tot = tot + lds4[w];
  __syncthreads();
  *total = tot;
  return out;
}

__device__ __forceinline__ float block_sum_f(float v, float* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += lds[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ double block_sum_d(double v, double* lds) {
  for (int m = 1; m < kWave; m <<= 1) v += shfl_xor_d(v, m);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += lds[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ SoftmaxPart block_merge(SoftmaxPart p, float sl, SoftmaxPart* lds) {
  p = wave_merge(p, sl);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = p;
  __syncthreads();
  SoftmaxPart t = lds[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) t = merge_parts(t, lds[w], sl);
  __syncthreads();
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
  __syncthreads();
  ArgMax t = lds[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) t = argmax_merge(t, lds[w]);
  __syncthreads();
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
  float cm = x[0];
#pragma unroll
  for (int i = 1; i + 1 < N; i += 2) cm = vmax3(cm, x[i], x[i + 1]);
  if constexpr ((N % 2) == 0) cm = vmax(cm, x[N - 1]);
  const float mn = vmax(s.m, cm);
  const float ms = (mn == -INFINITY) ? 0.0f : mn;
  const float msl = ms * sl;
  float e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = exp2_fast(__builtin_fmaf(x[i], sl, -msl));
  // pairwise sum of the group
#pragma unroll
  for (int w = 1; w < N; w <<= 1) {
#pragma unroll
    for (int i = 0; i + w < N; i += 2 * w) e[i] += e[i + w];
  }
  const float scale = exp2_fast(__builtin_fmaf(s.m, sl, -msl));
  s.z = __builtin_fmaf(s.z, scale, e[0]);
  s.m = mn;
}

// ---------------------------------------------------------------------------
// k_rowstats: one workgroup per (unit, segment); unit = r * (D_max + 1) + k.
template <typename E>
__global__ __launch_bounds__(kStatThreads) void k_rowstats(VerifyParams p) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  constexpr int G = VEC * kStatUnroll;  // values per thread per step
  __shared__ SoftmaxPart lds_sm[kStatThreads / kWave];
  __shared__ ArgMax lds_am[kStatThreads / kWave];

  const int seg = blockIdx.x % p.S1;
  const int unit = blockIdx.x / p.S1;
  const int r = unit / (p.D + 1);
  const int k = unit - r * (p.D + 1);
  const int n = p.depth[r];
  if (n < 0 || n > p.D || k > n) return;
  const float T = p.temperature[r];
  if (!temperature_ok(T)) return;
  const int64_t lo = (int64_t)seg * p.seg1;
  const int64_t hi = min(p.V, lo + (int64_t)p.seg1);
  const int64_t vhi = (hi > lo) ? lo + ((hi - lo) / VEC) * VEC : lo;
  const int64_t slot = (int64_t)unit * p.S1 + seg;
  const int tid = threadIdx.x;
  const S* prow = row_ptr<E>(p.target, p.target_row0[r] + k, p.stride);

  if (T == 0.0f) {
    // Arg max of the target row over the segment: per thread the best vector
    // (strictly greater keeps the earliest), then its first maximal element.
    float best = -INFINITY;
    int64_t bvec = -1;
    for (int64_t i = lo + (int64_t)tid * VEC; i < vhi; i += (int64_t)kStatThreads * VEC) {
      float x[VEC];
      E::unpack(load16(prow + i), x);
      float cm = x[0];
#pragma unroll
      for (int j = 1; j < VEC; ++j) cm = vmax(cm, x[j]);
      const bool up = cm > best;
      best = vmax(best, cm);
      bvec = up ? i : bvec;
    }
    ArgMax a{best, INT32_MAX};
    if (best == best && bvec >= 0) {
      float x[VEC];
      E::unpack(load16(prow + bvec), x);
#pragma unroll
      for (int j = VEC - 1; j >= 0; --j)
        if (x[j] == best) a.i = (int32_t)(bvec + j);
    }
    for (int64_t i = vhi + tid; i < hi; i += kStatThreads) {
      ArgMax t{E::load1(prow, i), (int32_t)i};
      a = argmax_merge(a, t);
    }
    a = block_argmax(a, lds_am);
    if (tid == 0) p.part_p[slot] = make_float2(a.v, __int_as_float(a.i));
    return;
  }

  const bool pair = k < n;
  const float sl = kLog2e / T;
  if (pair && p.draft == nullptr) return;  // flagged invalid by k_accept
  const S* qrow = pair ? row_ptr<E>(p.draft, p.draft_row0[r] + k, p.stride) : nullptr;
  SoftmaxPart sp{-INFINITY, 0.0f}, sq{-INFINITY, 0.0f};
  const int64_t step = (int64_t)kStatThreads * VEC;
  for (int64_t base = lo + (int64_t)tid * VEC; base < vhi; base += step * kStatUnroll) {
    // Loads past the segment read as a vector of -inf (masked: adds nothing).
    const uint4 pad = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
    uint4 pv[kStatUnroll], qv[kStatUnroll];
#pragma unroll
    for (int u = 0; u < kStatUnroll; ++u) {
      const int64_t i = base + u * step;
      pv[u] = (i < vhi) ? load16(prow + i) : pad;
      if (pair) qv[u] = (i < vhi) ? load16(qrow + i) : pad;
    }
    float x[G];
#pragma unroll
    for (int u = 0; u < kStatUnroll; ++u)
      E::unpack(pv[u], *reinterpret_cast<float(*)[VEC]>(&x[u * VEC]));
    softmax_group<G>(sp, x, sl);
    if (pair) {
#pragma unroll
      for (int u = 0; u < kStatUnroll; ++u)
        E::unpack(qv[u], *reinterpret_cast<float(*)[VEC]>(&x[u * VEC]));
      softmax_group<G>(sq, x, sl);
    }
  }
  for (int64_t i = vhi + tid; i < hi; i += kStatThreads) {
    float x1[1] = {E::load1(prow, i)};
    softmax_group<1>(sp, x1, sl);
    if (pair) {
      x1[0] = E::load1(qrow, i);
      softmax_group<1>(sq, x1, sl);
    }
  }
  sp = block_merge(sp, sl, lds_sm);
  if (pair) sq = block_merge(sq, sl, lds_sm);
  if (tid == 0) {
    p.part_p[slot] = make_float2(sp.m, sp.z);
    if (pair) p.part_q[slot] = make_float2(sq.m, sq.z);
  }
}

// Merge the S1 segment states of a row (fixed order).
__device__ __forceinline__ SoftmaxPart merge_row(const float2* parts, int64_t unit, int S1,
                                                 float sl) {
  SoftmaxPart s{-INFINITY, 0.0f};
  for (int j = 0; j < S1; ++j) {
    float2 v = parts[unit * S1 + j];
    s = merge_parts(s, SoftmaxPart{v.x, v.y}, sl);
  }
  return s;
}

__device__ __forceinline__ ArgMax merge_row_argmax(const float2* parts, int64_t unit, int S1) {
  ArgMax a{-INFINITY, INT32_MAX};
  for (int j = 0; j < S1; ++j) {
    float2 v = parts[unit * S1 + j];
    a = argmax_merge(a, ArgMax{v.x, __float_as_int(v.y)});
  }
  return a;
}

__device__ __forceinline__ bool finite_f(float x) { return x == x && x != INFINITY && x != -INFINITY; }

// ---------------------------------------------------------------------------
// k_alpha: sum_y min(p(y), q(y)) over one segment of a draft position's row
// pair, with the full-row normalisers merged from k_rowstats.
template <typename E>
__global__ __launch_bounds__(kStatThreads) void k_alpha(VerifyParams p) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  __shared__ float lds[kStatThreads / kWave];
  const int seg = blockIdx.x % p.S1;
  const int pos = blockIdx.x / p.S1;  // r * D + k
  const int r = pos / p.D;
  const int k = pos - r * p.D;
  const int n = p.depth[r];
  if (n < 0 || n > p.D || k >= n) return;
  const float T = p.temperature[r];
  if (!temperature_ok(T) || T == 0.0f || p.draft == nullptr) return;
  const float sl = kLog2e / T;
  const int64_t unit = (int64_t)r * (p.D + 1) + k;
  const SoftmaxPart sp = merge_row(p.part_p, unit, p.S1, sl);
  const SoftmaxPart sq = merge_row(p.part_q, unit, p.S1, sl);
  const int64_t slot = unit * p.S1 + seg;
  if (!finite_f(sp.m) || !finite_f(sq.m)) {
    if (threadIdx.x == 0) p.part_a[slot] = 0.0f;
    return;
  }
  // log2 p(y) = x sl - cp with cp = m sl + log2 z.
  const float cp = __builtin_fmaf(sp.m, sl, __log2f(sp.z));
  const float cq = __builtin_fmaf(sq.m, sl, __log2f(sq.z));
  const S* prow = row_ptr<E>(p.target, p.target_row0[r] + k, p.stride);
  const S* qrow = row_ptr<E>(p.draft, p.draft_row0[r] + k, p.stride);
  const int64_t lo = (int64_t)seg * p.seg1;
  const int64_t hi = min(p.V, lo + (int64_t)p.seg1);
  const int64_t vhi = (hi > lo) ? lo + ((hi - lo) / VEC) * VEC : lo;
  const int64_t step = (int64_t)kStatThreads * VEC;
  float acc = 0.0f;
  for (int64_t base = lo + (int64_t)threadIdx.x * VEC; base < vhi; base += step * kStatUnroll) {
    uint4 pv[kStatUnroll], qv[kStatUnroll];
    bool ok[kStatUnroll];
#pragma unroll
    for (int u = 0; u < kStatUnroll; ++u) {
      const int64_t i = base + u * step;
      ok[u] = i < vhi;
      if (ok[u]) {
        pv[u] = load16(prow + i);
        qv[u] = load16(qrow + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kStatUnroll; ++u) {
      if (!ok[u]) continue;
      float a[VEC], b[VEC];
      E::unpack(pv[u], a);
      E::unpack(qv[u], b);
      float e[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j)
        e[j] = exp2_fast(fminf(__builtin_fmaf(a[j], sl, -cp), __builtin_fmaf(b[j], sl, -cq)));
#pragma unroll
      for (int w = 1; w < VEC; w <<= 1) {
#pragma unroll
        for (int j = 0; j + w < VEC; j += 2 * w) e[j] += e[j + w];
      }
      acc += e[0];
    }
  }
  for (int64_t i = vhi + threadIdx.x; i < hi; i += kStatThreads) {
    const float a = E::load1(prow, i), b = E::load1(qrow, i);
    acc += exp2_fast(fminf(__builtin_fmaf(a, sl, -cp), __builtin_fmaf(b, sl, -cq)));
  }
  acc = block_sum_f(acc, lds);
  if (threadIdx.x == 0) p.part_a[slot] = acc;
}

// ---------------------------------------------------------------------------
// k_accept: one workgroup (2 wavefronts) per request.  Thread k handles
// target row k (k <= n) and, for k < n, draft row k and the accept test.
template <typename E>
__global__ __launch_bounds__(128) void k_accept(VerifyParams p) {
  using S = typename E::Storage;
  __shared__ uint32_t s_bits;
  __shared__ int s_tau;
  __shared__ float s_margin[128];
  const int r = blockIdx.x;
  const int k = threadIdx.x;
  const int D = p.D;
  const int n = p.depth[r];
  const float T = p.temperature[r];
  const uint32_t rid = p.request_id ? p.request_id[r] : (uint32_t)r;
  if (k == 0) s_bits = 0u;
  __syncthreads();

  uint32_t bits = 0u;
  if (n < 0 || n > D) bits |= SV_BIT_BAD_DEPTH;
  if (!temperature_ok(T)) bits |= SV_BIT_BAD_TEMPERATURE;
  const bool live = (bits == 0u) && k <= n;
  const int64_t unit = (int64_t)r * (D + 1) + k;

  bool keep = true;
  float margin = INFINITY;
  float sl = 0.0f;
  SoftmaxPart sp{0.0f, 1.0f}, sq{0.0f, 1.0f};
  ArgMax am{0.0f, 0};
  int32_t d = 0;
  if (live) {
    if (k < n) {
      d = p.tokens[(int64_t)r * D + k];
      if (d < 0 || (int64_t)d >= p.V) bits |= SV_BIT_BAD_TOKEN;
    }
    if (T == 0.0f) {
      am = merge_row_argmax(p.part_p, unit, p.S1);
      if (!finite_f(am.v)) bits |= SV_BIT_BAD_ROW;
      if (k < n) keep = (d == am.i);
    } else {
      sl = kLog2e / T;
      sp = merge_row(p.part_p, unit, p.S1, sl);
      if (!finite_f(sp.m)) bits |= SV_BIT_BAD_ROW;
      if (k < n) {
        if (p.draft == nullptr) {
          bits |= SV_BIT_BAD_ROW;
        } else {
          sq = merge_row(p.part_q, unit, p.S1, sl);
          if (!finite_f(sq.m)) bits |= SV_BIT_BAD_ROW;
        }
      }
      if (k < n && bits == 0u) {
        const S* prow = row_ptr<E>(p.target, p.target_row0[r] + k, p.stride);
        const S* qrow = row_ptr<E>(p.draft, p.draft_row0[r] + k, p.stride);
        const float pd = E::load1(prow, d), qd = E::load1(qrow, d);
        // log2 p(d) - log2 q(d), each as (x - m) sl - log2 z.
        const float lp = __builtin_fmaf(pd - sp.m, sl, -__log2f(sp.z));
        const float lq = __builtin_fmaf(qd - sq.m, sl, -__log2f(sq.z));
        const float ratio = exp2_fast(lp - lq);
        const Philox4 w = philox4x32_10((uint32_t)k, rid, p.step, 0u, p.seed_lo, p.seed_hi);
        const float u = u24(w.w[0]);
        keep = u < ratio;  // false when ratio is NaN (p(d) = q(d) = 0)
        margin = fabsf(u - ratio);
      }
    }
  }
  if (bits) atomicOr(&s_bits, bits);
  __syncthreads();
  const uint32_t all_bits = s_bits;

  if (all_bits != 0u) {  // nothing emitted for an invalid request
    if (k <= D) p.out_tokens[(int64_t)r * (D + 1) + k] = -1;
    if (k < D && p.alpha) p.alpha[(int64_t)r * D + k] = 0.0f;
    if (k == 0) {
      p.accepted_len[r] = 0;
      p.num_out[r] = 0;
      p.req[r].mode = kDrawNone;
      if (p.diag) p.diag[r] = sv_diag{INFINITY, INFINITY, all_bits, 0};
    }
    return;
  }

  // First rejection: ballot of rejected positions in wavefront 0 (k < n <= 64).
  if (k < kWave) {
    const uint64_t rejected = __ballot(k < n && !keep);
    if (k == 0) s_tau = rejected ? (int)__builtin_ctzll(rejected) : n;
  }
  s_margin[k] = (k < n) ? margin : INFINITY;
  __syncthreads();
  const int tau = s_tau;

  if (k <= D) {
    int32_t tok = -1;
    if (k < tau) tok = p.tokens[(int64_t)r * D + k];
    else if (k == tau && T == 0.0f) tok = am.i;
    p.out_tokens[(int64_t)r * (D + 1) + k] = tok;
  }
  if (k < D && p.alpha) {
    float a = 0.0f;
    if (k < n) {
      if (T == 0.0f) {
        a = keep ? 1.0f : 0.0f;
      } else {
        for (int j = 0; j < p.S1; ++j) a += p.part_a[unit * p.S1 + j];
      }
    }
    p.alpha[(int64_t)r * D + k] = a;
  }
  if (k == tau) {
    DrawState st;
    st.tau = tau;
    st.bits = 0u;
    st.need64 = 0;
    st.margin = INFINITY;
    if (T == 0.0f) {
      st.mode = kDrawNone;
    } else {
      st.mode = (tau < n) ? kDrawResidual : kDrawBonus;
      st.prow = p.target_row0[r] + tau;
      st.qrow = (tau < n) ? p.draft_row0[r] + tau : -1;
      st.sl = sl;
      st.T = T;
      st.mp = sp.m;
      st.lzp = __log2f(sp.z);
      st.zp = sp.z;
      st.mq = sq.m;
      st.lzq = __log2f(sq.z);
      const Philox4 w = philox4x32_10((uint32_t)tau, rid, p.step, 0u, p.seed_lo, p.seed_hi);
      st.u = u24(w.w[1]);
    }
    p.req[r] = st;
  }
  if (k == 0) {
    p.accepted_len[r] = tau;
    p.num_out[r] = tau + 1;
    if (p.diag) {
      float mm = INFINITY;
      for (int j = 0; j <= tau && j < n; ++j) mm = fminf(mm, s_margin[j]);
      p.diag[r] = sv_diag{mm, INFINITY, 0u, 0};
    }
  }
}

// ---------------------------------------------------------------------------
// Draw weights.  Residual: w(y) = max(0, p(y) - q(y)); bonus: w(y) = p(y).
template <typename E>
struct DrawRow32 {
  const typename E::Storage* prow;
  const typename E::Storage* qrow;  // null for a bonus draw
  float sl, mp, lzp, mq, lzq;
  __device__ __forceinline__ float w(float a, float b) const {
    const float pv = exp2_fast(__builtin_fmaf(a - mp, sl, -lzp));
    if (!qrow) return pv;
    const float qv = exp2_fast(__builtin_fmaf(b - mq, sl, -lzq));
    return fmaxf(pv - qv, 0.0f);
  }
  // The 8 weights of thread t in the tile starting at `tile` (0 past hi).
  __device__ __forceinline__ void weights(int64_t i0, int64_t hi, float (&out)[kDrawPerThread]) const {
#pragma unroll
    for (int j = 0; j < kDrawPerThread; ++j) {
      const int64_t i = i0 + j;
      if (i < hi) {
        const float a = E::load1(prow, i);
        const float b = qrow ? E::load1(qrow, i) : 0.0f;
        out[j] = w(a, b);
      } else {
        out[j] = 0.0f;
      }
    }
  }
};

template <typename E>
__device__ __forceinline__ DrawRow32<E> draw_row32(const VerifyParams& p, const DrawState& st) {
  DrawRow32<E> d;
  d.prow = row_ptr<E>(p.target, st.prow, p.stride);
  d.qrow = (st.mode == kDrawResidual) ? row_ptr<E>(p.draft, st.qrow, p.stride) : nullptr;
  d.sl = st.sl;
  d.mp = st.mp;
  d.lzp = st.lzp;
  d.mq = st.mq;
  d.lzq = st.lzq;
  return d;
}

// Sum of a thread's 8 weights, sequential (the canonical in-thread order).
template <typename T>
__device__ __forceinline__ T thread_sum(const T (&w)[kDrawPerThread]) {
  T s = w[0];
#pragma unroll
  for (int j = 1; j < kDrawPerThread; ++j) s = s + w[j];
  return s;
}

// k_draw_seg32: float32 mass of one draw segment = sequential sum over its
// tiles of the tile totals of the canonical block scan.
template <typename E>
__global__ __launch_bounds__(kDrawThreads) void k_draw_seg32(VerifyParams p) {
  __shared__ float lds4[kDrawThreads / kWave];
  const int r = blockIdx.y, seg = blockIdx.x;
  const DrawState st = p.req[r];
  if (st.mode == kDrawNone) return;
  const DrawRow32<E> dr = draw_row32<E>(p, st);
  const int64_t lo = (int64_t)seg * p.seg2, hi = min(p.V, lo + (int64_t)p.seg2);
  float total = 0.0f;
  for (int64_t tile = lo; tile < hi; tile += kDrawTile) {
    float w[kDrawPerThread];
    dr.weights(tile + (int64_t)threadIdx.x * kDrawPerThread, hi, w);
    float tt;
    block_inclusive_scan(thread_sum(w), lds4, &tt);
    total = total + tt;
  }
  if (threadIdx.x == 0) p.seg_w32[(int64_t)r * p.S2 + seg] = total;
}

// Locate the draw inside one segment: walk its tiles with the running
// cumulative mass C, scan the crossing tile, and return the first y with
// C(y) > t plus the distance from t to C(y-1) and C(y).  found = false if
// rounding left t beyond the segment (the caller then takes float64).
template <typename T>
struct LocateLds {
  T scan[kDrawThreads / kWave];
  T last[kDrawThreads / kWave];
  int wave_first[kDrawThreads / kWave];
  int found;
  int64_t y;
  T margin;
};

template <typename T, typename WeightsFn>
__device__ __forceinline__ void locate_in_segment(int64_t lo, int64_t hi, T c0, T t,
                                                  WeightsFn weights, LocateLds<T>& L) {
  T* lds4 = L.scan;
  T* lds_last = L.last;
  int* s_wave_first = L.wave_first;
  int* s_found = &L.found;
  int64_t* s_y = &L.y;
  T* s_margin = &L.margin;
  const int tid = threadIdx.x;
  T c = c0;
  if (tid == 0) *s_found = 0;
  __syncthreads();
  for (int64_t tile = lo; tile < hi; tile += kDrawTile) {
    T w[kDrawPerThread];
    const int64_t i0 = tile + (int64_t)tid * kDrawPerThread;
    weights(i0, hi, w);
    T tt;
    const T loc = thread_sum(w);
    const T incl = block_inclusive_scan(loc, lds4, &tt);
    // exclusive prefix = inclusive value of the previous thread
    T excl;
    if constexpr (sizeof(T) == 8) {
      int2 q = *reinterpret_cast<const int2*>(&incl);
      q.x = __shfl_up(q.x, 1);
      q.y = __shfl_up(q.y, 1);
      excl = *reinterpret_cast<T*>(&q);
    } else {
      excl = __shfl_up(incl, 1);
    }
    if ((tid & (kWave - 1)) == kWave - 1) lds_last[tid / kWave] = incl;
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) excl = (tid == 0) ? T(0) : lds_last[tid / kWave - 1];
    // Cumulative mass at each of this thread's elements.
    T run = excl;
    int first = -1;
    T before = c + excl, at = before;
#pragma unroll
    for (int j = 0; j < kDrawPerThread; ++j) {
      const T prev = c + run;
      run = run + w[j];
      const T cur = c + run;
      if (first < 0 && w[j] > T(0) && cur > t) {
        first = j;
        before = prev;
        at = cur;
      }
    }
    // The first thread (in thread order) holding a crossing wins.
    const uint64_t mask = __ballot(first >= 0);
    if ((tid & (kWave - 1)) == 0) s_wave_first[tid / kWave] = mask ? (int)__builtin_ctzll(mask) : -1;
    __syncthreads();
    int winner = -1;
    for (int wv = 0; wv < kDrawThreads / kWave; ++wv)
      if (s_wave_first[wv] >= 0) {
        winner = wv * kWave + s_wave_first[wv];
        break;
      }
    if (winner >= 0) {
      if (tid == winner) {
        *s_found = 1;
        *s_y = i0 + first;
        const T a = t - before, b = at - t;
        *s_margin = a < b ? a : b;
      }
      __syncthreads();
      return;
    }
    c = c + tt;
    __syncthreads();
  }
}

template <typename E>
__global__ __launch_bounds__(kDrawThreads) void k_draw_pick32(VerifyParams p) {
  __shared__ LocateLds<float> L;
  const int r = blockIdx.x;
  DrawState st = p.req[r];
  if (st.mode == kDrawNone) return;
  // Segment masses, total and the crossing segment (sequential, fixed order).
  float R = 0.0f;
  for (int j = 0; j < p.S2; ++j) R = R + p.seg_w32[(int64_t)r * p.S2 + j];
  const float t = st.u * R;
  int jstar = -1;
  float c0 = 0.0f;
  {
    float c = 0.0f;
    for (int j = 0; j < p.S2; ++j) {
      const float m = p.seg_w32[(int64_t)r * p.S2 + j];
      if (c + m > t) {
        jstar = j;
        c0 = c;
        break;
      }
      c = c + m;
    }
  }
  bool need64 = (p.flags & SV_FLAG_FORCE_FP64_DRAW) != 0u || !(R > 0.0f) || !(R < INFINITY) ||
                jstar < 0;
  float margin = 0.0f;
  int64_t y = -1;
  if (!need64) {
    const DrawRow32<E> dr = draw_row32<E>(p, st);
    const int64_t lo = (int64_t)jstar * p.seg2, hi = min(p.V, lo + (int64_t)p.seg2);
    locate_in_segment<float>(
        lo, hi, c0, t, [&](int64_t i0, int64_t h, float(&w)[kDrawPerThread]) { dr.weights(i0, h, w); },
        L);
    if (!L.found) {
      need64 = true;
    } else {
      y = L.y;
      margin = L.margin;
      if (!(margin >= kDrawMargin32)) need64 = true;
    }
  }
  if (threadIdx.x == 0) {
    if (need64) {
      p.req[r].need64 = 1;
      p.req[r].margin = margin;
    } else {
      p.out_tokens[(int64_t)r * (p.D + 1) + st.tau] = (int32_t)y;
      if (p.diag) p.diag[r].draw_margin = margin;
    }
  }
}

// ---------------------------------------------------------------------------
// Float64 recomputation of a draw: exact row maxima from the float32 pass,
// normalisers and weights in double with the temperature applied by division.
template <typename E>
struct DrawRow64 {
  const typename E::Storage* prow;
  const typename E::Storage* qrow;
  double T, mp, mq, lnzp, lnzq;
  bool unnormalised_p;  // weights exp((x - mp) / T) (residual mass was zero)
  __device__ __forceinline__ double w(double a, double b) const {
    if (unnormalised_p) return exp((a - mp) / T);
    const double pv = exp((a - mp) / T - lnzp);
    if (!qrow) return pv;
    const double qv = exp((b - mq) / T - lnzq);
    return pv > qv ? pv - qv : 0.0;
  }
  __device__ __forceinline__ void weights(int64_t i0, int64_t hi, double (&out)[kDrawPerThread]) const {
#pragma unroll
    for (int j = 0; j < kDrawPerThread; ++j) {
      const int64_t i = i0 + j;
      if (i < hi) {
        const double a = E::load1(prow, i);
        const double b = qrow ? (double)E::load1(qrow, i) : 0.0;
        out[j] = w(a, b);
      } else {
        out[j] = 0.0;
      }
    }
  }
};

template <typename E>
__global__ __launch_bounds__(kDrawThreads) void k_draw_z64(VerifyParams p) {
  __shared__ double lds[kDrawThreads / kWave];
  const int r = blockIdx.y, seg = blockIdx.x;
  const DrawState st = p.req[r];
  if (st.mode == kDrawNone || !st.need64) return;
  const typename E::Storage* prow = row_ptr<E>(p.target, st.prow, p.stride);
  const typename E::Storage* qrow =
      (st.mode == kDrawResidual) ? row_ptr<E>(p.draft, st.qrow, p.stride) : nullptr;
  const double T = st.T, mp = st.mp, mq = st.mq;
  const int64_t lo = (int64_t)seg * p.seg2, hi = min(p.V, lo + (int64_t)p.seg2);
  double zp = 0.0, zq = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kDrawThreads) {
    zp += exp(((double)E::load1(prow, i) - mp) / T);
    if (qrow) zq += exp(((double)E::load1(qrow, i) - mq) / T);
  }
  zp = block_sum_d(zp, lds);
  if (qrow) zq = block_sum_d(zq, lds);
  if (threadIdx.x == 0) {
    p.seg_zp64[(int64_t)r * p.S2 + seg] = zp;
    p.seg_zq64[(int64_t)r * p.S2 + seg] = zq;
  }
}

template <typename E>
__device__ __forceinline__ DrawRow64<E> draw_row64(const VerifyParams& p, const DrawState& st,
                                                   bool unnormalised_p) {
  DrawRow64<E> d;
  d.prow = row_ptr<E>(p.target, st.prow, p.stride);
  d.qrow = (st.mode == kDrawResidual && !unnormalised_p) ? row_ptr<E>(p.draft, st.qrow, p.stride)
                                                         : nullptr;
  d.T = st.T;
  d.mp = st.mp;
  d.mq = st.mq;
  d.lnzp = 0.0;
  d.lnzq = 0.0;
  d.unnormalised_p = unnormalised_p;
  return d;
}

template <typename E>
__device__ __forceinline__ void set_normalisers64(const VerifyParams& p, int r, DrawRow64<E>& d) {
  double zp = 0.0, zq = 0.0;
  for (int j = 0; j < p.S2; ++j) {
    zp += p.seg_zp64[(int64_t)r * p.S2 + j];
    zq += p.seg_zq64[(int64_t)r * p.S2 + j];
  }
  d.lnzp = log(zp);
  d.lnzq = (d.qrow != nullptr) ? log(zq) : 0.0;
}

template <typename E>
__global__ __launch_bounds__(kDrawThreads) void k_draw_seg64(VerifyParams p) {
  __shared__ double lds4[kDrawThreads / kWave];
  const int r = blockIdx.y, seg = blockIdx.x;
  const DrawState st = p.req[r];
  if (st.mode == kDrawNone || !st.need64) return;
  DrawRow64<E> dr = draw_row64<E>(p, st, false);
  set_normalisers64<E>(p, r, dr);
  const int64_t lo = (int64_t)seg * p.seg2, hi = min(p.V, lo + (int64_t)p.seg2);
  double total = 0.0;
  for (int64_t tile = lo; tile < hi; tile += kDrawTile) {
    double w[kDrawPerThread];
    dr.weights(tile + (int64_t)threadIdx.x * kDrawPerThread, hi, w);
    double tt;
    block_inclusive_scan(thread_sum(w), lds4, &tt);
    total = total + tt;
  }
  if (threadIdx.x == 0) p.seg_w64[(int64_t)r * p.S2 + seg] = total;
}

template <typename E>
__global__ __launch_bounds__(kDrawThreads) void k_draw_pick64(VerifyParams p) {
  __shared__ LocateLds<double> L;
  const int r = blockIdx.x;
  const DrawState st = p.req[r];
  if (st.mode == kDrawNone || !st.need64) return;
  const double u = st.u;
  double R = 0.0;
  for (int j = 0; j < p.S2; ++j) R = R + p.seg_w64[(int64_t)r * p.S2 + j];
  bool unnorm = !(R > 0.0);
  const double* segm = p.seg_w64;
  if (unnorm) {  // residual mass zero: draw from p (unnormalised weights)
    segm = p.seg_zp64;
    R = 0.0;
    for (int j = 0; j < p.S2; ++j) R = R + segm[(int64_t)r * p.S2 + j];
  }
  const double t = u * R;
  int jstar = -1;
  double c0 = 0.0;
  {
    double c = 0.0;
    int last_nonzero = -1;
    double c_last = 0.0;
    for (int j = 0; j < p.S2; ++j) {
      const double m = segm[(int64_t)r * p.S2 + j];
      if (m > 0.0) {
        last_nonzero = j;
        c_last = c;
      }
      if (c + m > t) {
        jstar = j;
        c0 = c;
        break;
      }
      c = c + m;
    }
    if (jstar < 0) {
      jstar = last_nonzero;
      c0 = c_last;
    }
  }
  int64_t y = -1;
  double margin = 0.0;
  if (jstar >= 0) {
    DrawRow64<E> dr = draw_row64<E>(p, st, unnorm);
    set_normalisers64<E>(p, r, dr);
    const int64_t lo = (int64_t)jstar * p.seg2, hi = min(p.V, lo + (int64_t)p.seg2);
    locate_in_segment<double>(
        lo, hi, c0, t, [&](int64_t i0, int64_t h, double(&w)[kDrawPerThread]) { dr.weights(i0, h, w); },
        L);
    if (L.found) {
      y = L.y;
      margin = L.margin;
    } else {
      // t rounded past the segment: the last token of non-zero weight in it.
      __shared__ unsigned long long s_last1;  // 1 + index of the last non-zero weight
      if (threadIdx.x == 0) s_last1 = 0ull;
      __syncthreads();
      for (int64_t i = lo + threadIdx.x; i < hi; i += kDrawThreads) {
        const double a = E::load1(dr.prow, i);
        const double b = dr.qrow ? (double)E::load1(dr.qrow, i) : 0.0;
        if (dr.w(a, b) > 0.0) atomicMax(&s_last1, (unsigned long long)(i + 1));
      }
      __syncthreads();
      y = (int64_t)s_last1 - 1;
      margin = 0.0;
    }
  }
  if (threadIdx.x == 0) {
    p.out_tokens[(int64_t)r * (p.D + 1) + st.tau] = (int32_t)y;
    if (p.diag) {
      p.diag[r].draw_margin = (float)margin;
      p.diag[r].bits |= SV_BIT_FP64_DRAW | (unnorm ? SV_BIT_RESIDUAL_ZERO : 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch sequence.
static void mark(const VerifyParams& p, int i, hipStream_t stream) {
  if (p.events) (void)hipEventRecord(static_cast<hipEvent_t>(p.events[i]), stream);
}

template <typename E>
static hipError_t launch_all(const VerifyParams& p, hipStream_t stream) {
  const int U = p.B * (p.D + 1);
  mark(p, 0, stream);
  hipLaunchKernelGGL(k_rowstats<E>, dim3((unsigned)(U * p.S1)), dim3(kStatThreads), 0, stream, p);
  mark(p, 1, stream);
  if (p.alpha && p.D > 0)
    hipLaunchKernelGGL(k_alpha<E>, dim3((unsigned)(p.B * p.D * p.S1)), dim3(kStatThreads), 0,
                       stream, p);
  mark(p, 2, stream);
  hipLaunchKernelGGL(k_accept<E>, dim3((unsigned)p.B), dim3(128), 0, stream, p);
  mark(p, 3, stream);
  hipLaunchKernelGGL(k_draw_seg32<E>, dim3((unsigned)p.S2, (unsigned)p.B), dim3(kDrawThreads), 0,
                     stream, p);
  hipLaunchKernelGGL(k_draw_pick32<E>, dim3((unsigned)p.B), dim3(kDrawThreads), 0, stream, p);
  hipLaunchKernelGGL(k_draw_z64<E>, dim3((unsigned)p.S2, (unsigned)p.B), dim3(kDrawThreads), 0,
                     stream, p);
  hipLaunchKernelGGL(k_draw_seg64<E>, dim3((unsigned)p.S2, (unsigned)p.B), dim3(kDrawThreads), 0,
                     stream, p);
  hipLaunchKernelGGL(k_draw_pick64<E>, dim3((unsigned)p.B), dim3(kDrawThreads), 0, stream, p);
  mark(p, 4, stream);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyParams& p, hipStream_t stream) {
  return (p.dtype == SV_DTYPE_BF16) ? launch_all<Bf16>(p, stream) : launch_all<F32>(p, stream);
}

}  // namespace sv
