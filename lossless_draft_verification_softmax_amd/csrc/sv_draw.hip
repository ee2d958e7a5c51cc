// sv_draw.hip -- the float64 recompute of the draws that the float32 draw
// of the accept-and-draw kernel (sv_verify.hip) leaves too close to a CDF
// boundary: inverse-CDF draw from normalize(max(0, p - q)) after a
// rejection, or from p after a fully accepted block (the standard
// rejection-sampling rule behind the lossless verification of the
// tradepoint.io page, "Why one universal drafter underperforms").
//
// The row is cut into tiles of 2048 elements (one 16-byte load of bf16 per
// thread of a 256-thread workgroup).  A tile's mass is the last value of a
// fixed-order block scan of its weights, so the pass that finds the crossing
// tile and the pass that scans inside it agree bit for bit.
//   k_draw_tile64   one float64 pass over the rows of queued requests: tile
//                   normaliser partials and the one-pass split of the tile
//                   residual masses
//   k_draw_pick64   float64 tile masses (from the split, or directly where
//                   it is not certain), then the float64 pick
// The float64 kernels walk the queue on a fixed grid, so an empty queue costs
// one short dispatch each.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_drawrow.hpp"
#include "sv_shard.hpp"

namespace sv {

constexpr int kDrawThreads = 256;
constexpr int kQueueGrid = 2048;

// Fixed-order block scan (Hillis-Steele in each wavefront, wave totals in
// order).  Returns the inclusive value; *total gets the block total.
template <typename T>
__device__ __forceinline__ T scan256(T v, T* lds, T* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T o;
    if constexpr (sizeof(T) == 8) {
      int2 q = *reinterpret_cast<int2*>(&v);
      q.x = __shfl_up(q.x, d);
      q.y = __shfl_up(q.y, d);
      o = *reinterpret_cast<T*>(&q);
    } else {
      o = __shfl_up(v, d);
    }
    if (lane >= d) v = v + o;
  }
  if (lane == kWave - 1) lds[wave] = v;
  __syncthreads();
  T base = T(0);
  for (int w = 0; w < wave; ++w) base = base + lds[w];
  const T out = (wave == 0) ? v : base + v;
  T tot = lds[0];
  for (int w = 1; w < kDrawThreads / kWave; ++w) tot = tot + lds[w];
  __syncthreads();
  *total = tot;
  return out;
}

template <typename T>
__device__ __forceinline__ T shfl_up1(T v) {
  if constexpr (sizeof(T) == 8) {
    int2 q = *reinterpret_cast<int2*>(&v);
    q.x = __shfl_up(q.x, 1);
    q.y = __shfl_up(q.y, 1);
    return *reinterpret_cast<T*>(&q);
  } else {
    return __shfl_up(v, 1);
  }
}

template <typename T>
__device__ __forceinline__ T block_sum256(T v, T* lds) {
  for (int m = 1; m < kWave; m <<= 1) {
    if constexpr (sizeof(T) == 8) v += shfl_xor_d(v, m);
    else v += __shfl_xor(v, m);
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  T t = T(0);
  for (int w = 0; w < kDrawThreads / kWave; ++w) t = t + lds[w];
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// Float64 weights: the temperature is applied as a multiplication by the
// float64 reciprocal of T (one extra rounding, about 1e-16 relative, where a
// division would cost ten float64 operations per element); the normalisers
// are float64 sums of exp((x - max) / T).
template <typename E, bool SH>
struct Weights64 {
  RowView<E, SH> prow, qrow;
  bool has_q;
  double invT, mp, mq, lnzp, lnzq;
  bool unnormalised;  // w = exp((x - mp) / T): residual mass was zero
  __device__ __forceinline__ void operator()(int64_t i0, int64_t hi, double (&w)[kPer]) const {
    float a[kPer];
    load8<E, SH>(prow, i0, hi, a);
    if (unnormalised || !has_q) {
      const double off = unnormalised ? 0.0 : lnzp;
#pragma unroll
      for (int j = 0; j < kPer; ++j) w[j] = exp(((double)a[j] - mp) * invT - off);
      return;
    }
    float b[kPer];
    load8<E, SH>(qrow, i0, hi, b);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const double pv = exp(((double)a[j] - mp) * invT - lnzp);
      const double qv = exp(((double)b[j] - mq) * invT - lnzq);
      w[j] = pv > qv ? pv - qv : 0.0;
    }
  }
};

template <typename T>
__device__ __forceinline__ T sum8(const T (&w)[kPer]) {
  T s = w[0];
#pragma unroll
  for (int j = 1; j < kPer; ++j) s = s + w[j];
  return s;
}

// Mass of tile `tile` of a row: the block-scan total of the thread sums.
template <typename T, typename W>
__device__ __forceinline__ T tile_mass(const W& weights, int64_t tile, int64_t V, T* lds) {
  const int64_t lo = tile * kDrawTile;
  const int64_t hi = min(V, lo + (int64_t)kDrawTile);
  T w[kPer];
  weights(lo + (int64_t)threadIdx.x * kPer, hi, w);
  T tot;
  scan256<T>(sum8(w), lds, &tot);
  return tot;
}

struct PickResult {
  int64_t y;
  double margin;
  double R;  // total of the tile masses
  int found;
};

template <typename T>
struct PickLds {
  T scan[kDrawThreads / kWave];
  T last[kDrawThreads / kWave];
  int wave_first[kDrawThreads / kWave];
  int64_t y;
  double margin;
  int found;
  int tile;
  T c0, t;
};

// The draw given per-tile masses: scan the masses (rounds of 256 tiles, carry
// in order) for the total R and the crossing tile, then scan inside it.  The
// first y with C(y) > t = u * R wins; margin = min(t - C(y-1), C(y) - t).
// When the tiles fit one round (S2 <= 256) the one scan gives both the total
// and every tile's inclusive value.
template <typename T, typename W>
__device__ PickResult pick(const T* masses, int64_t S2, int64_t V, T u, const W& weights,
                           PickLds<T>& L) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  if (tid == 0) {
    L.found = 0;
    L.tile = -1;
  }
  T carry = T(0);
  T m1 = T(0), incl1 = T(0);  // this thread's tile (single round)
  for (int64_t base = 0; base < S2; base += kDrawThreads) {
    const T m = (base + tid < S2) ? masses[base + tid] : T(0);
    T tot;
    const T incl = scan256<T>(m, L.scan, &tot);
    m1 = m;
    incl1 = incl;
    carry = carry + tot;
  }
  const T R = carry;
  const T t = u * R;
  // crossing tile: the first tile whose inclusive cumulative mass exceeds t
  carry = T(0);
  for (int64_t base = 0; base < S2; base += kDrawThreads) {
    T m = m1, incl = incl1, tot = R;
    if (S2 > kDrawThreads) {
      m = (base + tid < S2) ? masses[base + tid] : T(0);
      incl = carry + scan256<T>(m, L.scan, &tot);
    }
    T excl = shfl_up1(incl);
    // exclusive value across wave boundaries: previous thread's inclusive
    if (lane == kWave - 1) L.last[tid / kWave] = incl;
    __syncthreads();
    if (lane == 0) excl = (tid == 0) ? carry : L.last[tid / kWave - 1];
    const bool cross = (base + tid < S2) && m > T(0) && incl > t;
    const uint64_t mask = __ballot(cross);
    if (lane == 0) L.wave_first[tid / kWave] = mask ? (int)__builtin_ctzll(mask) : -1;
    __syncthreads();
    int winner = -1;
    for (int w = 0; w < kDrawThreads / kWave; ++w)
      if (L.wave_first[w] >= 0) {
        winner = w * kWave + L.wave_first[w];
        break;
      }
    if (winner >= 0) {
      if (tid == winner) {
        L.tile = (int)(base + tid);
        L.c0 = excl;
      }
      __syncthreads();
      break;
    }
    carry = carry + tot;
    __syncthreads();
  }
  PickResult res{-1, 0.0, (double)R, 0};
  const int tile = L.tile;
  if (tile < 0) return res;  // t at or past the total: undecided
  const T c0 = L.c0;
  const int64_t lo = (int64_t)tile * kDrawTile;
  const int64_t hi = min(V, lo + (int64_t)kDrawTile);
  T w[kPer];
  const int64_t i0 = lo + (int64_t)tid * kPer;
  weights(i0, hi, w);
  T tot;
  const T incl = scan256<T>(sum8(w), L.scan, &tot);
  T excl = shfl_up1(incl);
  if (lane == kWave - 1) L.last[tid / kWave] = incl;
  __syncthreads();
  if (lane == 0) excl = (tid == 0) ? T(0) : L.last[tid / kWave - 1];
  T run = excl;
  int first = -1;
  T before = T(0), at = T(0);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const T prev = c0 + run;
    run = run + w[j];
    const T cur = c0 + run;
    if (first < 0 && w[j] > T(0) && cur > t) {
      first = j;
      before = prev;
      at = cur;
    }
  }
  const uint64_t mask = __ballot(first >= 0);
  if (lane == 0) L.wave_first[tid / kWave] = mask ? (int)__builtin_ctzll(mask) : -1;
  __syncthreads();
  int winner = -1;
  for (int wv = 0; wv < kDrawThreads / kWave; ++wv)
    if (L.wave_first[wv] >= 0) {
      winner = wv * kWave + L.wave_first[wv];
      break;
    }
  if (winner >= 0 && tid == winner) {
    L.found = 1;
    L.y = i0 + first;
    const T a = t - before, b = at - t;
    L.margin = (double)(a < b ? a : b);
  }
  __syncthreads();
  res.found = L.found;
  res.y = L.y;
  res.margin = L.margin;
  return res;
}

// ---------------------------------------------------------------------------
template <typename E, bool SH>
__device__ __forceinline__ Weights64<E, SH> weights64(const VerifyParams& p, const DrawState& st,
                                                  bool unnormalised) {
  Weights64<E, SH> w;
  w.has_q = st.mode == kDrawResidual && !unnormalised;
  w.prow = row_view<E, SH>(p, false, st.prow);
  w.qrow = row_view<E, SH>(p, true, w.has_q ? st.qrow : 0);
  w.invT = 1.0 / (double)st.T;
  w.mp = st.mp;
  w.mq = st.mq;
  w.lnzp = 0.0;
  w.lnzq = 0.0;
  w.unnormalised = unnormalised;
  return w;
}

// Float64 pass over one tile of a queued draw row: the normaliser partials
// sum exp((x - max) / T) of p and q, and the one-pass split of the residual
// mass.  With rho = Zq / Zp, an element's residual weight is
// max(0, ep rho - eq) / Zq (ep, eq the unnormalised exponentials).  Against
// the float32 estimate rho_e of rho, d = ep rho_e - eq is computed with one
// rounding (fma); elements with d > tau ep rho_e are certainly positive,
// those with d < -tau ep rho_e certainly not, once |rho / rho_e - 1| <= tau / 2
// holds (checked by the pick).  Over the certain-positive elements the tile
// keeps D = sum d and A = sum ep, and its residual mass is then
// (D + (rho - rho_e) A) / Zq, free of cancellation.  Equal logits (a = b,
// common once both rows are rounded to bfloat16) have eq = kappa ep with one
// kappa = exp((mp - mq) / T) for the whole row, so they are kept apart as
// S = sum ep and add S max(0, (Zq - kappa Zp) / (Zp Zq)).  The few other
// elements in between keep their (ep, eq) (up to kDrawKeep64 per tile, in
// element order) and the pick adds their exact weights; a tile with more is
// recomputed directly.
constexpr double kTau64 = 1e-4;

// log2(Zq / Zp) from the float32 row states, with Z = sum 2^((x - m) sl): each
// log2 sum lz is taken against the integer reference R(m), so each adds its
// offset R(m) - m sl (exact in float64, as the product of two floats is).
__device__ __forceinline__ double log2_ratio_exact(const DrawState& st) {
  const double op = (double)ref_of(st.mp, st.sl) - (double)st.mp * (double)st.sl;
  const double oq = (double)ref_of(st.mq, st.sl) - (double)st.mq * (double)st.sl;
  return ((double)st.lzq + oq) - ((double)st.lzp + op);
}

template <typename E, bool SH>
__global__ __launch_bounds__(kDrawThreads) void k_draw_tile64(VerifyParams p) {
  __shared__ double lds[kDrawThreads / kWave][5];
  __shared__ int32_t ldsu[kDrawThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t items = (int64_t)(*p.fb_count) * p.S2;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int r = p.fb_list[it / p.S2];
    const int64_t tile = it % p.S2;
    const DrawState st = p.req[r];
    const bool residual = st.mode == kDrawResidual;
    const double invT = 1.0 / (double)st.T;
    const double rho_e = residual ? exp2(log2_ratio_exact(st)) : 0.0;
    const int64_t lo = tile * kDrawTile, hi = min(p.V, lo + (int64_t)kDrawTile);
    const int64_t i0 = lo + (int64_t)threadIdx.x * kPer;
    float a[kPer], b[kPer];
    load8<E, SH>(row_view<E, SH>(p, false, st.prow), i0, hi, a);
    if (residual) load8<E, SH>(row_view<E, SH>(p, true, st.qrow), i0, hi, b);
    double zp = 0.0, zq = 0.0, D = 0.0, A = 0.0, S = 0.0;
    uint32_t kmask = 0u;  // elements kept for the pick (their ep, eq recomputed below)
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const double ep = exp(((double)a[j] - (double)st.mp) * invT);
      zp += ep;
      if (residual) {
        const double eq = exp(((double)b[j] - (double)st.mq) * invT);
        zq += eq;
        const double d = fma(ep, rho_e, -eq);
        const double tol = kTau64 * ep * rho_e;
        if (a[j] == b[j]) {
          S += ep;
        } else if (d > tol) {
          D += d;
          A += ep;
        } else if (d >= -tol && (ep > 0.0 || eq > 0.0)) {
          kmask |= 1u << j;
        }
      }
    }
    // kept elements: positions by an exclusive scan of the counts in thread
    // order, so the list is in element order
    const int32_t U = __builtin_popcount(kmask);
    int32_t incl = U;
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) ldsu[wave] = incl;
    __syncthreads();
    int32_t base = 0, total = 0;
    for (int w = 0; w < kDrawThreads / kWave; ++w) {
      if (w < wave) base += ldsu[w];
      total += ldsu[w];
    }
    base += incl - U;
    const int64_t o = (int64_t)r * p.S2 + tile;
    if (total <= kDrawKeep64 && kmask != 0u) {
      double* keep = p.seg_e64 + o * (kDrawKeep64 * 2);
      int32_t pos = base;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if ((kmask >> j) & 1u) {
          keep[2 * pos] = exp(((double)a[j] - (double)st.mp) * invT);
          keep[2 * pos + 1] = exp(((double)b[j] - (double)st.mq) * invT);
          ++pos;
        }
      }
    }
    // block sums in a fixed order
    for (int m = 1; m < kWave; m <<= 1) {
      zp += shfl_xor_d(zp, m);
      zq += shfl_xor_d(zq, m);
      D += shfl_xor_d(D, m);
      A += shfl_xor_d(A, m);
      S += shfl_xor_d(S, m);
    }
    __syncthreads();
    if (lane == 0) {
      lds[wave][0] = zp;
      lds[wave][1] = zq;
      lds[wave][2] = D;
      lds[wave][3] = A;
      lds[wave][4] = S;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double t[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
      for (int w = 0; w < kDrawThreads / kWave; ++w)
        for (int k = 0; k < 5; ++k) t[k] += lds[w][k];
      p.seg_zp64[o] = t[0];
      p.seg_zq64[o] = t[1];
      p.seg_w64[o] = t[2];
      p.seg_a64[o] = t[3];
      p.seg_t64[o] = t[4];
      p.seg_u32[o] = total;
    }
    __syncthreads();
  }
}

// Full-row float64 normalisers of both rows from the tile partials (the same
// fixed-order tree for each), in one block reduction.
__device__ __forceinline__ void merge_z64(const double* pp, const double* pq, int64_t S2,
                                          double (*lds)[2], double& zp, double& zq) {
  double a = 0.0, b = 0.0;
  for (int64_t j = threadIdx.x; j < S2; j += kDrawThreads) {
    a += pp[j];
    if (pq) b += pq[j];
  }
  for (int m = 1; m < kWave; m <<= 1) {
    a += shfl_xor_d(a, m);
    b += shfl_xor_d(b, m);
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) {
    lds[wave][0] = a;
    lds[wave][1] = b;
  }
  __syncthreads();
  zp = 0.0;
  zq = 0.0;
  for (int w = 0; w < kDrawThreads / kWave; ++w) {
    zp += lds[w][0];
    zq += lds[w][1];
  }
  __syncthreads();
}

template <typename E, bool SH>
__global__ __launch_bounds__(kDrawThreads) void k_draw_pick64(VerifyParams p) {
  __shared__ PickLds<double> L;
  __shared__ double lds[kDrawThreads / kWave];
  __shared__ double lds2[kDrawThreads / kWave][2];
  __shared__ int s_redo[kDrawThreads];
  __shared__ double s_mass[kDrawThreads];
  const int r = blockIdx.x;
  const DrawState st = p.req[r];
  if (st.mode == kDrawNone || !st.need64) return;
  const bool residual = st.mode == kDrawResidual;
  const int64_t ro = (int64_t)r * p.S2;
  // Tile masses stay in LDS when the row has at most one round of tiles.
  double* masses = p.S2 <= kDrawThreads ? s_mass : p.seg_w64 + ro;
  // The first round's split results are loaded together with the
  // normaliser partials: one memory round trip before the masses.
  const int64_t t0 = threadIdx.x;
  const bool have0 = residual && t0 < p.S2;
  int32_t nk0 = 0;
  double d0 = 0.0, a0 = 0.0, s0 = 0.0;
  double2 kv0[kDrawKeep64];
  if (have0) {
    nk0 = p.seg_u32[ro + t0];
    d0 = p.seg_w64[ro + t0];
    a0 = p.seg_a64[ro + t0];
    s0 = p.seg_t64[ro + t0];
    const double2* keep = reinterpret_cast<const double2*>(p.seg_e64 + (ro + t0) * (kDrawKeep64 * 2));
#pragma unroll
    for (int k = 0; k < kDrawKeep64; ++k) kv0[k] = keep[k];
  }
  double Zp, Zq;
  merge_z64(p.seg_zp64 + ro, residual ? p.seg_zq64 + ro : nullptr, p.S2, lds2, Zp, Zq);
  if (!residual) Zq = 1.0;
  Weights64<E, SH> w = weights64<E, SH>(p, st, false);
  w.lnzp = log(Zp);
  w.lnzq = log(Zq);
  // Tile masses: from the one-pass split where it is certain, else directly.
  const double rho = Zq / Zp;
  const double rho_e = residual ? exp2(log2_ratio_exact(st)) : 0.0;
  const bool split_ok = residual && (p.flags & SV_FLAG_EXACT_FP64_MASSES) == 0u &&
                        fabs(rho / rho_e - 1.0) <= 0.5 * kTau64;
  // residual weight per unit of ep of an equal-logit pair
  const double kappa = exp(((double)st.mp - (double)st.mq) * w.invT);
  const double g_tie = fmax(0.0, (Zq - kappa * Zp) / (Zp * Zq));
  const double izp = 1.0 / Zp, izq = 1.0 / Zq;
  for (int64_t base = 0; base < p.S2; base += kDrawThreads) {
    const int64_t t = base + threadIdx.x;
    int redo = 0;
    if (t < p.S2) {
      const int64_t o = ro + t;
      if (!residual) {
        masses[t] = p.seg_zp64[o] / Zp;
      } else if (split_ok) {
        int32_t nk = nk0;
        double d = d0, a = a0, sv = s0;
        double2 kv[kDrawKeep64];
        if (base == 0) {
#pragma unroll
          for (int k = 0; k < kDrawKeep64; ++k) kv[k] = kv0[k];
        } else {
          nk = p.seg_u32[o];
          d = p.seg_w64[o];
          a = p.seg_a64[o];
          sv = p.seg_t64[o];
          // the whole list is loaded at once (entries past nk are unused)
          const double2* keep = reinterpret_cast<const double2*>(p.seg_e64 + o * (kDrawKeep64 * 2));
#pragma unroll
          for (int k = 0; k < kDrawKeep64; ++k) kv[k] = keep[k];
        }
        if (nk <= kDrawKeep64) {
          double m = (d + (rho - rho_e) * a) * izq + sv * g_tie;
#pragma unroll
          for (int k = 0; k < kDrawKeep64; ++k)
            if (k < nk) m += fmax(0.0, kv[k].x * izp - kv[k].y * izq);
          masses[t] = m;
        } else {
          redo = 1;
        }
      } else {
        redo = 1;
      }
    }
    s_redo[threadIdx.x] = redo;
    // usually no tile needs a direct recompute: skip the walk over the flags
    if (__syncthreads_or(redo)) {
      for (int k = 0; k < kDrawThreads && base + k < p.S2; ++k) {
        if (!s_redo[k]) continue;  // uniform: every thread reads the same flag
        const double m = tile_mass<double>(w, base + k, p.V, lds);
        if (threadIdx.x == 0) masses[base + k] = m;
      }
    }
    __syncthreads();
  }
  // The pick scans the tile masses once for the residual mass R and the
  // crossing tile.  R = 0 (p = q to float64 precision): draw from p, from the
  // unnormalised tile partials.
  PickResult res = pick<double>(masses, p.S2, p.V, (double)st.u, w, L);
  const bool unnorm = !(res.R > 0.0);
  if (unnorm) {
    const Weights64<E, SH> wu = weights64<E, SH>(p, st, true);
    res = pick<double>(p.seg_zp64 + (int64_t)r * p.S2, p.S2, p.V, (double)st.u, wu, L);
  }
  if (!res.found) {
    // t rounded to or past the total: the last token of non-zero weight.
    __shared__ unsigned long long s_last1;
    if (threadIdx.x == 0) s_last1 = 0ull;
    __syncthreads();
    const Weights64<E, SH> wl = unnorm ? weights64<E, SH>(p, st, true) : w;
    for (int64_t tile = 0; tile < p.S2; ++tile) {
      const int64_t lo = tile * kDrawTile, hi = min(p.V, lo + (int64_t)kDrawTile);
      const int64_t i0 = lo + (int64_t)threadIdx.x * kPer;
      double e[kPer];
      wl(i0, hi, e);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (e[j] > 0.0) atomicMax(&s_last1, (unsigned long long)(i0 + j + 1));
    }
    __syncthreads();
    res.y = (int64_t)s_last1 - 1;
    res.margin = 0.0;
  }
  if (threadIdx.x == 0) {
    p.out_tokens[(int64_t)r * (p.D + 1) + st.tau] = (int32_t)res.y;
    if (p.diag) {
      p.diag[r].draw_margin = (float)res.margin;
      p.diag[r].bits |= SV_BIT_FP64_DRAW | (unnorm ? SV_BIT_RESIDUAL_ZERO : 0u);
    }
  }
}

template <typename E, bool SH>
static void launch_draw_t(const VerifyParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((k_draw_tile64<E, SH>), dim3(kQueueGrid), dim3(kDrawThreads), 0, stream, p);
  hipLaunchKernelGGL((k_draw_pick64<E, SH>), dim3((unsigned)p.B), dim3(kDrawThreads), 0, stream, p);
}

void launch_draw(const VerifyParams& p, hipStream_t stream) {
  const bool sh = p.nshard > 1;
  if (p.dtype == SV_DTYPE_BF16) {
    if (sh) launch_draw_t<Bf16, true>(p, stream);
    else launch_draw_t<Bf16, false>(p, stream);
  } else {
    if (sh) launch_draw_t<F32, true>(p, stream);
    else launch_draw_t<F32, false>(p, stream);
  }
}

}  // namespace sv
