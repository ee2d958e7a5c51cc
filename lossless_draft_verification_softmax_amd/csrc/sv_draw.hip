// sv_draw.hip -- the float64 recompute of the draws that the float32 draw
// of the accept-and-draw kernel (sv_verify.hip) leaves too close to a CDF
// boundary: inverse-CDF draw from normalize(max(0, p - q)) after a
// rejection, or from p after a fully accepted block (the standard
// rejection-sampling rule behind the lossless verification of the
// tradepoint.io page, "Why one universal drafter underperforms").
//
// The row is cut into tiles of 2048 elements (one 16-byte load of bf16 per
// thread of a 256-thread workgroup).
//   k_draw_tile64   one float64 pass over the (queued draw, tile) items: tile
//                   normaliser partials and the one-pass split of the tile
//                   residual masses; one more workgroup, when asked for,
//                   writes the batch's acceptance statistics meanwhile
//                   (sv_stats.hpp)
//   k_draw_pick64   one workgroup per queued draw: tile masses from the
//                   partials, the crossing tile and the scan inside it
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_drawrow.hpp"
#include "sv_exp64.hpp"
#include "sv_params.hpp"
#include "sv_shard.hpp"
#include "sv_stats.hpp"

namespace sv {

constexpr int kDrawThreads = 256;
// Tile-pass workgroups per CU: all resident at once (four waves per SIMD at
// up to 128 registers per lane).
constexpr int kTileBlocksPerCu = 4;

// Float64 sum over the wavefront, the same value on every lane: the fixed
// tree of wave_allreduce (quad, 8-lane and 16-lane mirrors, then the row and
// half swaps), both 32-bit halves of an operand moving together.
template <int kCtrl>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, kCtrl, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), kCtrl, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Float64 sum over each 16-lane row, the same value on every lane of the row.
__device__ __forceinline__ double row_sum_d(double v) {
  v = v + dpp_d<kDppQuadXor1>(v);
  v = v + dpp_d<kDppQuadXor2>(v);
  v = v + dpp_d<kDppHalfMirror>(v);
  return v + dpp_d<kDppMirror>(v);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v = row_sum_d(v);
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  v = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
      __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
  const uint64_t c = __builtin_bit_cast(uint64_t, v);
  lo = __builtin_amdgcn_permlane32_swap((uint32_t)c, (uint32_t)c, false, false);
  hi = __builtin_amdgcn_permlane32_swap((uint32_t)(c >> 32), (uint32_t)(c >> 32), false, false);
  return __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
         __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}

// DPP moves with a row mask (rows left out read 0).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double dpp_d_rows(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, kCtrl, kRowMask, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), kCtrl, kRowMask, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Inclusive float64 scan over the wavefront in a fixed order: Hillis-Steele
// steps inside each 16-lane row (row shifts by 1, 2, 4, 8), then row 0's
// total into row 1 and row 2's into row 3 (broadcast of lane 15 of a row),
// then the total of rows 0-1 into rows 2 and 3 (broadcast of lane 31).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143, kDppWaveShr1 = 0x138;
__device__ __forceinline__ double wave_scan_d(double v) {
  const int lane = threadIdx.x & (kWave - 1), r = lane & 15;
  double o = dpp_d<kDppRowShr1>(v);
  if (r >= 1) v = v + o;
  o = dpp_d<kDppRowShr2>(v);
  if (r >= 2) v = v + o;
  o = dpp_d<kDppRowShr4>(v);
  if (r >= 4) v = v + o;
  o = dpp_d<kDppRowShr8>(v);
  if (r >= 8) v = v + o;
  o = dpp_d_rows<kDppRowBcast15, 0xA>(v);
  if (lane & 16) v = v + o;
  o = dpp_d_rows<kDppRowBcast31, 0xC>(v);
  if (lane >= 32) v = v + o;
  return v;
}

// Block-level exchanges of the pick go through two sets of LDS slots used in
// turn (`buf`, flipped by each exchange): every exchange has one barrier
// between its writes and its reads, so the set an exchange writes was last
// read before the previous exchange's barrier.
struct PickLds {
  double wtot[2][kDrawThreads / kWave];  // wavefront totals of a block scan
  int first[2][kDrawThreads / kWave];    // first crossing lane of each wavefront, or -1
  double c0[2][kDrawThreads / kWave];    // its exclusive cumulative value
  int64_t y[2][kDrawThreads / kWave];    // (scan in a tile) its token
  double margin[2][kDrawThreads / kWave];
};

// Block scan of one float64 per thread: returns the inclusive value, with
// *excl the previous thread's inclusive value (0 for thread 0) and *total the
// block total.  The wavefront totals are added in order, the same way for
// the inclusive and the exclusive values, so a thread's *excl equals the
// previous thread's return value bit for bit.
__device__ __forceinline__ double block_scan_d(double v, PickLds& L, int& buf, double* excl,
                                               double* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const double incl = wave_scan_d(v);
  const double prev = dpp_d<kDppWaveShr1>(incl);  // lane 0 reads 0
  if (lane == kWave - 1) L.wtot[buf][wave] = incl;
  __syncthreads();
  double base = 0.0, tot = 0.0;
  for (int w = 0; w < kDrawThreads / kWave; ++w) {
    const double x = L.wtot[buf][w];
    if (w < wave) base = base + x;
    tot = tot + x;
  }
  buf ^= 1;
  *total = tot;
  if (wave == 0) {
    *excl = lane == 0 ? 0.0 : prev;
    return incl;
  }
  *excl = lane == 0 ? base : base + prev;
  return base + incl;
}

// Block total of one float64 per thread (the total of block_scan_d).
__device__ __forceinline__ double block_sum_d(double v, PickLds& L, int& buf) {
  double excl, tot;
  block_scan_d(v, L, buf, &excl, &tot);
  return tot;
}

// ---------------------------------------------------------------------------
// Float64 weights: the temperature is applied as a multiplication by the
// float64 reciprocal of T (one extra rounding, about 1e-16 relative, where a
// division would cost ten float64 operations per element); an element's
// unnormalised exponentials are ep = exp((a - mp) / T), eq = exp((b - mq) / T),
// their arguments taken in one fma as a / T + (-m / T) (the rounding of
// -m / T scales a whole row by one factor, which its normaliser cancels),
// and its weight max(0, ep / Zp - eq / Zq) (residual draw) or ep / Zp (bonus
// draw), with the float64 normalisers Zp = sum ep, Zq = sum eq applied as
// reciprocals.  Every path that weighs an element (the kept near-ties, the
// float32 draw's tile, a directly recomputed tile) uses this one formula.
template <typename E, bool SH>
struct Weights64 {
  RowView<E, SH> prow, qrow;
  bool has_q;         // residual draw: w = max(0, p - q); else w = p
  double invT, cp, cq;  // exponent arguments fma(x, 1/T, c): c = -m / T of the row
  double izp, izq;    // 1 / Zp, 1 / Zq (izp = 1: the unnormalised p of a zero residual)
  const double* tab;  // 2^(j/256) table of exp64_tab (LDS)
  // weights from the unnormalised exponentials
  __device__ __forceinline__ double weight(double ep, double eq) const {
    if (!has_q) return ep * izp;
    const double pv = ep * izp, qv = eq * izq;
    return pv > qv ? pv - qv : 0.0;
  }
  // weights of eight logits a (target) and b (draft; read only if has_q)
  __device__ __forceinline__ void from(const float (&a)[kPer], const float (&b)[kPer],
                                       double (&w)[kPer]) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const double ep = exp64_tab(fma((double)a[j], invT, cp), tab);
      const double eq = has_q ? exp64_tab(fma((double)b[j], invT, cq), tab) : 0.0;
      w[j] = weight(ep, eq);
    }
  }
  __device__ __forceinline__ void operator()(int64_t i0, int64_t hi, double (&w)[kPer]) const {
    float a[kPer], b[kPer];
    load8_pair<E, SH>(prow, qrow, has_q, i0, hi, a, b);
    from(a, b, w);
  }
};

template <typename E, bool SH>
__device__ __forceinline__ Weights64<E, SH> weights64(const VerifyParams& p, const DrawJob& jb,
                                                      bool unnormalised, double izp, double izq,
                                                      const double* tab) {
  Weights64<E, SH> w;
  w.has_q = jb.mode == kDrawResidual && !unnormalised;
  w.prow = row_view<E, SH>(p, false, jb.prow);
  w.qrow = row_view<E, SH>(p, true, w.has_q ? jb.qrow : 0);
  w.invT = jb.invT;
  w.cp = -(double)jb.mp * jb.invT;
  w.cq = -(double)jb.mq * jb.invT;
  w.izp = unnormalised ? 1.0 : izp;
  w.izq = izq;
  w.tab = tab;
  return w;
}

__device__ __forceinline__ double sum8(const double (&w)[kPer]) {
  double s = w[0];
#pragma unroll
  for (int j = 1; j < kPer; ++j) s = s + w[j];
  return s;
}

// The crossing tile of a draw given the per-tile masses: one scan of the
// masses (rounds of 256 tiles, carry in order) for the total R, and
// t = u R; the crossing tile is the first tile of non-zero mass whose
// inclusive cumulative mass exceeds t.  tile = -1 when t is at or past the
// total (rounding).  With at most 256 tiles the one scan gives both the total
// and every tile's inclusive value.
struct TileFind {
  int tile;
  double c0;  // cumulative mass before the tile
  double t;
  double R;
};

__device__ TileFind find_tile(const double* masses, int64_t S2, double u, PickLds& L, int& buf) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  double carry = 0.0;
  double m1 = 0.0, incl1 = 0.0, excl1 = 0.0;  // this thread's tile (single round)
  for (int64_t base = 0; base < S2; base += kDrawThreads) {
    const double m = (base + tid < S2) ? masses[base + tid] : 0.0;
    double tot;
    incl1 = block_scan_d(m, L, buf, &excl1, &tot);
    m1 = m;
    carry = carry + tot;
  }
  const double R = carry;
  const double t = u * R;
  carry = 0.0;
  TileFind f{-1, 0.0, t, R};
  for (int64_t base = 0; base < S2; base += kDrawThreads) {
    double m = m1, incl = incl1, excl = excl1, tot = R;
    if (S2 > kDrawThreads) {
      m = (base + tid < S2) ? masses[base + tid] : 0.0;
      incl = carry + block_scan_d(m, L, buf, &excl, &tot);
      excl = carry + excl;
    }
    const bool cross = (base + tid < S2) && m > 0.0 && incl > t;
    const uint64_t mask = __ballot(cross);
    const int fl = mask ? (int)__builtin_ctzll(mask) : -1;
    if (lane == 0) L.first[buf][wave] = fl;
    if (lane == fl) L.c0[buf][wave] = excl;
    __syncthreads();
    for (int w = 0; w < kDrawThreads / kWave; ++w) {
      const int fw = L.first[buf][w];
      if (fw >= 0) {
        f.tile = (int)(base + w * kWave + fw);
        f.c0 = L.c0[buf][w];
        break;
      }
    }
    buf ^= 1;
    if (f.tile >= 0) break;  // uniform
    carry = carry + tot;
  }
  return f;
}

// Inside the crossing tile: a block scan of the weights (thread i holding
// elements i0 .. i0 + 7) from c0; the first y with C(y) > t wins, with
// margin = min(t - C(y-1), C(y) - t).
struct InTile {
  int found;
  int64_t y;
  double margin;
};

__device__ InTile scan_in_tile(const double (&w)[kPer], int64_t i0, double c0, double t,
                               PickLds& L, int& buf) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  double excl, tot;
  block_scan_d(sum8(w), L, buf, &excl, &tot);
  double run = excl;
  int first = -1;
  double before = 0.0, at = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const double prev = c0 + run;
    run = run + w[j];
    const double cur = c0 + run;
    if (first < 0 && w[j] > 0.0 && cur > t) {
      first = j;
      before = prev;
      at = cur;
    }
  }
  const uint64_t mask = __ballot(first >= 0);
  const int fl = mask ? (int)__builtin_ctzll(mask) : -1;
  if (lane == 0) L.first[buf][wave] = fl;
  if (lane == fl) {
    L.y[buf][wave] = i0 + first;
    const double a = t - before, b = at - t;
    L.margin[buf][wave] = a < b ? a : b;
  }
  __syncthreads();
  InTile r{0, -1, 0.0};
  for (int wv = 0; wv < kDrawThreads / kWave; ++wv) {
    if (L.first[buf][wv] >= 0) {
      r = InTile{1, L.y[buf][wv], L.margin[buf][wv]};
      break;
    }
  }
  buf ^= 1;
  return r;
}

// ---------------------------------------------------------------------------
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

struct Draw64Lds {
  double tab[kExp64Table];  // 2^(j/256) for exp64_tab
  // sums over the 16-lane rows of a tile pass item, and the kept-element
  // counts of its wavefronts; two sets (item parity), so that one barrier
  // per item separates a set's writes from its last reads
  double red[2][kDrawThreads / 16][5];
  int32_t redu[2][kDrawThreads / kWave];
  double z2[kDrawThreads / kWave][2];
  double mass[kDrawThreads];  // tile masses of a row of at most 256 tiles
  int redo[kDrawThreads];
  PickLds pk;
  unsigned long long last1;
};

// The exponential table goes to LDS one entry per thread: the entry is
// loaded at kernel entry, together with the kernel's first other loads, and
// stored before the first barrier (every exp64_tab comes after it).
static_assert(kExp64Table == kDrawThreads, "one table entry per thread");
__device__ __forceinline__ double exp_table_entry() { return kExp2Frac[threadIdx.x]; }

// Exponentials of the float32 draw's tile, kept by the tile pass for the pick:
// [entry][row][element j of a thread][thread].
__device__ __forceinline__ double* hint_exps(const VerifyParams& p, int slot, int row) {
  return p.seg_h64 + ((int64_t)slot * 2 + row) * kDrawTile;
}

// This thread's eight elements of tile `tile` of a queued draw's rows.
template <typename E, bool SH>
__device__ __forceinline__ void tile_load(const VerifyParams& p, const DrawJob& jb, int64_t tile,
                                          Raw8<E>& raw) {
  const int64_t lo = tile * kDrawTile, hi = min(p.V, lo + (int64_t)kDrawTile);
  load_raw8<E, SH>(row_view<E, SH>(p, false, jb.prow), row_view<E, SH>(p, true, jb.qrow),
                   jb.mode == kDrawResidual, lo + (int64_t)threadIdx.x * kPer, hi, raw);
}

template <typename E, bool SH>
__device__ __forceinline__ void tile_pass(const VerifyParams& p, const DrawJob& jb, int slot,
                                          int64_t tile, const Raw8<E>& raw, int buf, Draw64Lds& L) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t o = (int64_t)slot * p.S2 + tile;
  const bool residual = jb.mode == kDrawResidual;
  const bool hinted = jb.y32 >= 0 && (int64_t)jb.y32 / kDrawTile == tile;
  const double invT = jb.invT, rho_e = jb.rho_e;
  const double cp = -(double)jb.mp * invT, cq = -(double)jb.mq * invT;
  const double tau_rho = kTau64 * rho_e;
  const int64_t lo = tile * kDrawTile, hi = min(p.V, lo + (int64_t)kDrawTile);
  const int64_t i0 = lo + (int64_t)threadIdx.x * kPer;
  float a[kPer], b[kPer];
  unpack_raw8<E, SH>(raw, row_view<E, SH>(p, false, jb.prow), row_view<E, SH>(p, true, jb.qrow),
                     residual, i0, hi, a, b);
  double* hp = hint_exps(p, slot, 0) + threadIdx.x;
  double* hq = hint_exps(p, slot, 1) + threadIdx.x;
  double zp = 0.0, zq = 0.0, D = 0.0, A = 0.0, S = 0.0;
  uint32_t kmask = 0u;  // elements kept for the pick (their ep, eq recomputed below)
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const double ep = exp64_tab(fma((double)a[j], invT, cp), L.tab);
    zp += ep;
    if (hinted) hp[j * kDrawThreads] = ep;
    if (residual) {
      const double eq = exp64_tab(fma((double)b[j], invT, cq), L.tab);
      zq += eq;
      if (hinted) hq[j * kDrawThreads] = eq;
      // the element's class, without branches (the sums of the other
      // classes add an exact 0)
      const double d = fma(ep, rho_e, -eq);
      const double tol = tau_rho * ep;
      const bool same = a[j] == b[j];
      const bool pos = !same && d > tol;
      // (ep = 0 weighs max(0, -eq) = 0: never kept)
      const bool keep = !same && !pos && d >= -tol && ep > 0.0;
      S += same ? ep : 0.0;
      D += pos ? d : 0.0;
      A += pos ? ep : 0.0;
      kmask |= (uint32_t)keep << j;
    }
  }
  // kept elements: positions in element order (a lane's eight elements are
  // consecutive; lanes, then wavefronts, in order), from one ballot per
  // element slot; usually no element of the wavefront is kept
  int32_t before = 0, wave_kept = 0;
  if (__ballot(kmask != 0u) != 0ull) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint64_t bal = __ballot((kmask >> j) & 1u);
      before += (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      wave_kept += __builtin_popcountll(bal);
    }
  }
  zp = row_sum_d(zp);
  if (residual) {
    zq = row_sum_d(zq);
    D = row_sum_d(D);
    A = row_sum_d(A);
    S = row_sum_d(S);
  }
  if ((lane & 15) == 0) {
    const int row = wave * (kWave / 16) + lane / 16;
    L.red[buf][row][0] = zp;
    L.red[buf][row][1] = zq;
    L.red[buf][row][2] = D;
    L.red[buf][row][3] = A;
    L.red[buf][row][4] = S;
    if (lane == 0) L.redu[buf][wave] = wave_kept;
  }
  __syncthreads();
  int32_t base = before, total = 0;
  for (int w = 0; w < kDrawThreads / kWave; ++w) {
    const int32_t c = L.redu[buf][w];
    if (w < wave) base += c;
    total += c;
  }
  if (total <= kDrawKeep64 && kmask != 0u) {
    double* keep = p.seg_e64 + o * (kDrawKeep64 * 2);
    int32_t pos = base;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if ((kmask >> j) & 1u) {
        keep[2 * pos] = exp64_tab(fma((double)a[j], invT, cp), L.tab);
        keep[2 * pos + 1] = exp64_tab(fma((double)b[j], invT, cq), L.tab);
        ++pos;
      }
    }
  }
  // block sums in a fixed order, one value per lane of the first wavefront
  if (threadIdx.x < 6) {
    const int k = threadIdx.x;
    if (k == 5) {
      p.seg_u32[o] = total;
    } else {
      double t = 0.0;
      for (int w = 0; w < kDrawThreads / 16; ++w) t += L.red[buf][w][k];
      double* dst = k == 0 ? p.seg_zp64 : k == 1 ? p.seg_zq64 : k == 2 ? p.seg_w64
                                                 : k == 3 ? p.seg_a64 : p.seg_t64;
      dst[o] = t;
    }
  }
}

// Mass of tile `tile` of a row, recomputed directly: the block total of the
// thread sums of its float64 weights.
template <typename W>
__device__ __forceinline__ double tile_mass(const W& weights, int64_t tile, int64_t V, PickLds& L,
                                            int& buf) {
  const int64_t lo = tile * kDrawTile;
  const int64_t hi = min(V, lo + (int64_t)kDrawTile);
  double w[kPer];
  weights(lo + (int64_t)threadIdx.x * kPer, hi, w);
  return block_sum_d(sum8(w), L, buf);
}

// The float64 draw of queue entry `slot`: full-row normalisers from the tile
// partials, the tile masses (from the split where it is certain, else
// directly), the crossing tile and the scan inside it.  The exponentials of
// the float32 draw's tile, which the tile pass kept, are loaded at the start
// together with the partials: the crossing tile is almost always that one,
// as the two draws differ by less than the float32 error.
template <typename E, bool SH>
__device__ void pick64(const VerifyParams& p, const DrawJob& jb, int slot, Draw64Lds& L) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const bool residual = jb.mode == kDrawResidual;
  const int64_t S2 = p.S2;
  const int64_t ro = (int64_t)slot * S2;
  const int64_t htile = jb.y32 >= 0 ? (int64_t)jb.y32 / kDrawTile : -1;
  int buf = 0;  // LDS slot set of the next block exchange (PickLds)
  double hep[kPer], heq[kPer];
  if (htile >= 0) {
    const double* hp = hint_exps(p, slot, 0) + tid;
    const double* hq = hint_exps(p, slot, 1) + tid;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      hep[j] = hp[j * kDrawThreads];
      heq[j] = residual ? hq[j * kDrawThreads] : 0.0;
    }
  }
  // the first round of tile partials, and the request's diagnostic bits
  // (so that the last step waits on no load)
  const bool have0 = tid < S2;
  double zp0 = 0.0, zq0 = 0.0, d0 = 0.0, a0 = 0.0, s0 = 0.0;
  int32_t nk0 = 0;
  if (have0) {
    zp0 = p.seg_zp64[ro + tid];
    if (residual) {
      zq0 = p.seg_zq64[ro + tid];
      d0 = p.seg_w64[ro + tid];
      a0 = p.seg_a64[ro + tid];
      s0 = p.seg_t64[ro + tid];
      nk0 = p.seg_u32[ro + tid];
    }
  }
  const uint32_t bits0 = (p.diag && tid == 0) ? p.diag[jb.r].bits : 0u;
  // full-row normalisers: thread sums over the rounds, then a fixed-order tree
  double zps = zp0, zqs = zq0;
  for (int64_t j = tid + kDrawThreads; j < S2; j += kDrawThreads) {
    zps += p.seg_zp64[ro + j];
    if (residual) zqs += p.seg_zq64[ro + j];
  }
  zps = wave_sum_d(zps);
  zqs = wave_sum_d(zqs);
  if (lane == 0) {
    L.z2[wave][0] = zps;
    L.z2[wave][1] = zqs;
  }
  __syncthreads();
  // the first four kept elements of each tile of the first round (read
  // whatever their count, only the first nk are used), in flight while the
  // normalisers are inverted
  double2 kv0[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) kv0[k] = make_double2(0.0, 0.0);
  if (have0 && residual) {
    const double2* keep = reinterpret_cast<const double2*>(p.seg_e64 + (ro + tid) * (kDrawKeep64 * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k) kv0[k] = keep[k];
  }
  double Zp = 0.0, Zq = 0.0;
  for (int w = 0; w < kDrawThreads / kWave; ++w) {
    Zp += L.z2[w][0];
    Zq += L.z2[w][1];
  }
  if (!residual) Zq = 1.0;
  const double izp = 1.0 / Zp, izq = 1.0 / Zq;
  const Weights64<E, SH> w = weights64<E, SH>(p, jb, false, izp, izq, L.tab);
  // (equal logits a = b have eq / ep = kappa = exp(cq - cp) for the whole row)
  const double kappa = exp64_tab(w.cq - w.cp, L.tab);
  // tile masses: from the one-pass split where it is certain, else directly
  double* masses = S2 <= kDrawThreads ? L.mass : p.seg_w64 + ro;
  const double rho = Zq * izp;
  const double rho_e = jb.rho_e;
  const bool split_ok = residual && (p.flags & SV_FLAG_EXACT_FP64_MASSES) == 0u &&
                        fabs(rho - rho_e) <= 0.5 * kTau64 * rho_e;
  const double g_tie = fmax(0.0, izp - kappa * izq);
  for (int64_t base = 0; base < S2; base += kDrawThreads) {
    const int64_t t = base + tid;
    int redo = 0;
    if (t < S2) {
      const int64_t o = ro + t;
      if (!residual) {
        masses[t] = (base == 0 ? zp0 : p.seg_zp64[o]) * izp;
      } else if (split_ok) {
        int32_t nk = nk0;
        double d = d0, a = a0, sv = s0;
        if (base != 0) {
          nk = p.seg_u32[o];
          d = p.seg_w64[o];
          a = p.seg_a64[o];
          sv = p.seg_t64[o];
        }
        if (nk <= kDrawKeep64) {
          double m = (d + (rho - rho_e) * a) * izq + sv * g_tie;
          // the kept elements, four loads at a time, in element order
          const double2* keep = reinterpret_cast<const double2*>(p.seg_e64 + o * (kDrawKeep64 * 2));
          for (int k0 = 0; k0 < nk; k0 += 4) {
            double2 kv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              kv[k] = (base == 0 && k0 == 0) ? kv0[k]
                      : (k0 + k < nk)        ? keep[k0 + k]
                                             : make_double2(0.0, 0.0);
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (k0 + k < nk) m += w.weight(kv[k].x, kv[k].y);
          }
          masses[t] = m;
        } else {
          redo = 1;
        }
      } else {
        redo = 1;
      }
    }
    L.redo[tid] = redo;
    // usually no tile needs a direct recompute: skip the walk over the flags
    // (the barrier of __syncthreads_or also publishes the masses)
    if (__syncthreads_or(redo)) {
      for (int k = 0; k < kDrawThreads && base + k < S2; ++k) {
        if (!L.redo[k]) continue;  // uniform: every thread reads the same flag
        const double m = tile_mass(w, base + k, p.V, L.pk, buf);
        if (tid == 0) masses[base + k] = m;
      }
      __syncthreads();
    }
  }
  // R = 0 (p = q to float64 precision): draw from p, from the unnormalised
  // tile partials.
  TileFind f = find_tile(masses, S2, (double)jb.u, L.pk, buf);
  const bool unnorm = !(f.R > 0.0);
  if (unnorm) f = find_tile(p.seg_zp64 + ro, S2, (double)jb.u, L.pk, buf);
  const Weights64<E, SH> wd = unnorm ? weights64<E, SH>(p, jb, true, 1.0, 1.0, L.tab) : w;
  InTile res{0, -1, 0.0};
  if (f.tile >= 0) {
    const int64_t lo = (int64_t)f.tile * kDrawTile, hi = min(p.V, lo + (int64_t)kDrawTile);
    const int64_t i0 = lo + (int64_t)tid * kPer;
    double wv[kPer];
    if (f.tile == htile) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) wv[j] = wd.weight(hep[j], heq[j]);
    } else {
      wd(i0, hi, wv);
    }
    res = scan_in_tile(wv, i0, f.c0, f.t, L.pk, buf);
  }
  if (!res.found) {
    // t rounded to or past the total: the last token of non-zero weight.
    if (tid == 0) L.last1 = 0ull;
    __syncthreads();
    for (int64_t tile = 0; tile < S2; ++tile) {
      const int64_t lo = tile * kDrawTile, hi = min(p.V, lo + (int64_t)kDrawTile);
      const int64_t i0 = lo + (int64_t)tid * kPer;
      double e[kPer];
      wd(i0, hi, e);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (e[j] > 0.0) atomicMax(&L.last1, (unsigned long long)(i0 + j + 1));
    }
    __syncthreads();
    res.y = (int64_t)L.last1 - 1;
    res.margin = 0.0;
  }
  if (tid == 0) {
    p.out_tokens[(int64_t)jb.r * (p.D + 1) + jb.tau] = (int32_t)res.y;
    if (p.diag) {
      p.diag[jb.r].draw_margin = (float)res.margin;
      p.diag[jb.r].bits = bits0 | SV_BIT_FP64_DRAW | (unnorm ? SV_BIT_RESIDUAL_ZERO : 0u);
    }
  }
}

// Tile pass: the (queue entry, tile) items are dealt to a grid of
// kTileBlocksPerCu workgroups per CU, all resident at once, item it to
// workgroup it mod grid.  Each workgroup issues the loads of its next item
// before it works on the current one.  Its first loads (the queue entries
// of its first two items, the queue length and its exponential table entry)
// go out together at entry; an entry is used only once the length shows
// that it is queued.  An empty queue costs one short dispatch.  Item
// indices fit 32 bits (the host bounds B times the tiles per row).
template <typename E, bool SH>
__device__ __forceinline__ void tile_items(const VerifyParams& p, uint32_t wg, uint32_t G,
                                           Draw64Lds& L) {
  const uint32_t S2 = (uint32_t)p.S2, cap = (uint32_t)p.B * S2;
  uint32_t it = wg;
  DrawJob jb{}, jn{};
  if (it < cap) jb = p.fb_jobs[it / S2];
  if (it + G < cap) jn = p.fb_jobs[(it + G) / S2];
  const double tab = exp_table_entry();
  const uint32_t items = (uint32_t)*p.fb_count * S2;
  // (the table load is issued before the exit test, not sunk below it)
  asm volatile("" ::"v"(tab));
  if (it >= items) return;
  L.tab[threadIdx.x] = tab;
  Raw8<E> raw;
  tile_load<E, SH>(p, jb, it % S2, raw);
  __syncthreads();
  for (int buf = 0; it < items; it += G, buf ^= 1) {
    // the next item's loads (the current item's again past the end, so
    // that every address is valid and no branch splits the loads)
    const uint32_t nx = it + G;
    const bool more = nx < items;
    Raw8<E> rawn;
    tile_load<E, SH>(p, more ? jn : jb, more ? nx % S2 : it % S2, rawn);
    DrawJob jnn{};
    if (nx + G < items) jnn = p.fb_jobs[(nx + G) / S2];
    const uint32_t slot = it / S2;
    tile_pass<E, SH>(p, jb, (int)slot, (int64_t)(it - slot * S2), raw, buf, L);
    raw = rawn;
    jb = jn;
    jn = jnn;
  }
}

// When the caller asked for the batch's acceptance statistics (accepted
// lengths and rates are final once k_accept_draw has run), workgroup 0,
// dispatched first, writes them while the tile workgroups 1, 2, ... run;
// the one tile workgroup that finds no free slot at first is the last, which
// has the fewest items.
template <typename E, bool SH>
__global__ __launch_bounds__(kDrawThreads, kTileBlocksPerCu) void k_draw_tile64(VerifyParams p) {
  __shared__ union {
    Draw64Lds d;
    StatsLds s;
  } L;
  warm_params(p);
  const bool stats = p.stats_expected_len || p.stats_per_depth || p.stats_summary;
  if (stats && blockIdx.x == 0) {
    accept_stats_block<kDrawThreads / kWave, 4>(p.depth, p.alpha, p.accepted_len, p.B, p.D,
                                                p.stats_expected_len, p.stats_per_depth,
                                                p.stats_summary, L.s);
    return;
  }
  const uint32_t first = stats ? 1u : 0u;
  tile_items<E, SH>(p, blockIdx.x - first, gridDim.x - first, L.d);
}

// Pick: workgroup j draws queue entry j.
template <typename E, bool SH>
__global__ __launch_bounds__(kDrawThreads) void k_draw_pick64(VerifyParams p) {
  __shared__ Draw64Lds L;
  warm_params(p);
  const int slot = blockIdx.x;
  const DrawJob jb = p.fb_jobs[slot];
  const double tab = exp_table_entry();
  asm volatile("" ::"v"(tab));
  if (slot >= *p.fb_count) return;
  L.tab[threadIdx.x] = tab;  // visible after pick64's first barrier
  pick64<E, SH>(p, jb, slot, L);
}

template <typename E, bool SH>
static void launch_draw_t(const VerifyParams& p, int cus, hipStream_t stream) {
  const bool stats = p.stats_expected_len || p.stats_per_depth || p.stats_summary;
  hipLaunchKernelGGL((k_draw_tile64<E, SH>), dim3(cus * kTileBlocksPerCu + (stats ? 1 : 0)),
                     dim3(kDrawThreads), 0, stream, p);
  hipLaunchKernelGGL((k_draw_pick64<E, SH>), dim3((unsigned)p.B), dim3(kDrawThreads), 0, stream, p);
}

void launch_draw(const VerifyParams& p, int cus, hipStream_t stream) {
  const bool sh = p.nshard > 1;
  if (p.dtype == SV_DTYPE_BF16) {
    if (sh) launch_draw_t<Bf16, true>(p, cus, stream);
    else launch_draw_t<Bf16, false>(p, cus, stream);
  } else {
    if (sh) launch_draw_t<F32, true>(p, cus, stream);
    else launch_draw_t<F32, false>(p, cus, stream);
  }
}

}  // namespace sv
