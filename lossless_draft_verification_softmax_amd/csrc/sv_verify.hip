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
//   k_plan          the work list (sv_rowpass.hip).
//   k_rowteam       row statistics and acceptance rates, per slice of every
//   (k_rowpass)     row (sv_rowteam.hip; the streaming pass in sv_rowpass.hip).
//   k_accept_draw   one workgroup per request: the accept test per position,
//                   wavefront ballot + first set bit = tau, emitted drafts,
//                   alpha, and the float32 inverse-CDF draw of the correction
//                   / bonus token from the slices' masses and one slice scan.
//   k_draw_tile64,  float64 recompute of the draws left within the float32
//   k_draw_pick64   error of a CDF boundary (sv_draw.hip).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_drawrow.hpp"
#include "sv_internal.hpp"
#include "sv_shard.hpp"

namespace sv {


// Merge the nseg segment states of a row (fixed order).  The slot loads are
// issued kMergeChunk at a time so that a row costs one memory latency per
// chunk rather than one per slot.
constexpr int kMergeChunk = 16;

// v holds the first chunk of slots, loaded by the caller (entries past nseg
// set to the empty state); later chunks are loaded here.
__device__ __forceinline__ SoftmaxPart merge_row(const float2 (&v0)[kMergeChunk],
                                                 const float2* parts, int64_t unit, int S1,
                                                 int nseg, float sl) {
  SoftmaxPart s{-INFINITY, 0.0f};
#pragma unroll
  for (int i = 0; i < kMergeChunk; ++i) s = merge_parts(s, SoftmaxPart{v0[i].x, v0[i].y}, sl);
  const float2* row = parts + unit * S1;
  for (int j0 = kMergeChunk; j0 < nseg; j0 += kMergeChunk) {
    float2 v[kMergeChunk];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i)
      v[i] = (j0 + i < nseg) ? row[j0 + i] : make_float2(-INFINITY, 0.0f);
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) s = merge_parts(s, SoftmaxPart{v[i].x, v[i].y}, sl);
  }
  return s;
}

__device__ __forceinline__ ArgMax merge_row_argmax(const float2 (&v0)[kMergeChunk],
                                                   const float2* parts, int64_t unit, int S1) {
  ArgMax a{-INFINITY, INT32_MAX};
#pragma unroll
  for (int i = 0; i < kMergeChunk; ++i) a = argmax_merge(a, ArgMax{v0[i].x, __float_as_int(v0[i].y)});
  const float2* row = parts + unit * S1;
  for (int j0 = kMergeChunk; j0 < S1; j0 += kMergeChunk) {
    float2 v[kMergeChunk];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i)
      v[i] = (j0 + i < S1) ? row[j0 + i] : make_float2(-INFINITY, __int_as_float(INT32_MAX));
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i)
      a = argmax_merge(a, ArgMax{v[i].x, __float_as_int(v[i].y)});
  }
  return a;
}

__device__ __forceinline__ bool finite_f(float x) { return x == x && x != INFINITY && x != -INFINITY; }

// ---------------------------------------------------------------------------
// k_accept_draw: one 1024-thread workgroup per request.
//
// Accept (threads 0..D): thread k takes target row k (k <= n) and, for
// k < n, draft row k and the accept test; a wavefront ballot of the rejected
// positions and its first set bit give tau; the emitted drafts, alpha and the
// diagnostics follow.
//
// Draw (T > 0, the whole workgroup), float32, without a pass over the row:
// the row pass left, for every slice s of the draw row (a team member's
// slice, or a streaming segment), the slice's state of the target row and,
// for a row pair, its sum alpha_s of min(p, q).  The slice's share of p is
// P_s = z_s 2^(R(m_s) - log2 Z_p), so its residual mass is
// max(0, P_s - alpha_s) (P_s for a bonus draw).  A wavefront scan of those
// masses gives R and the slice holding t = u R; only that slice is then
// read and scanned element by element.  The token is written when its CDF
// margin is at least kDrawMargin32 (which covers the float32 errors of the
// slice masses and of the scan); otherwise, or when rounding leaves t outside
// the slice, the request joins the float64 queue (sv_draw.hip).
constexpr int kAcceptDrawThreads = 1024;
constexpr int kAcceptDrawWaves = kAcceptDrawThreads / kWave;
constexpr int kChunk = kAcceptDrawThreads * kPer;  // elements per scan span
constexpr int kScanSpans = 2;                       // spans per scan round

struct AcceptDrawLds {
  uint32_t bits;
  int tau;
  float margin[kWave + 1];
  DrawState st;
  int slice;       // crossing slice, or -1
  float c0, t;     // cumulative mass before the slice, target u R
  // per scan round (two sets used in turn, so that one barrier per
  // exchange suffices) and span: wavefront totals, and each wavefront's
  // first crossing element with the cumulative masses around it
  float wtot[2][kScanSpans][kAcceptDrawWaves];
  int wfirst[2][kScanSpans][kAcceptDrawWaves];
  int32_t wy[2][kScanSpans][kAcceptDrawWaves];
  float wbefore[2][kScanSpans][kAcceptDrawWaves], wat[2][kScanSpans][kAcceptDrawWaves];
};

// Inclusive float32 scan over the wavefront in a fixed order, by DPP moves:
// Hillis-Steele steps inside each 16-lane row, then row 0's total into row
// 1 and row 2's into row 3 (broadcast of lane 15 of a row), then the total of
// rows 0-1 into rows 2 and 3 (broadcast of lane 31).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ float wave_scan_f(float v) {
  const int lane = threadIdx.x & (kWave - 1), r = lane & 15;
  float o = dpp_f<0x111>(v);  // row_shr:1
  if (r >= 1) v += o;
  o = dpp_f<0x112>(v);        // row_shr:2
  if (r >= 2) v += o;
  o = dpp_f<0x114>(v);        // row_shr:4
  if (r >= 4) v += o;
  o = dpp_f<0x118>(v);        // row_shr:8
  if (r >= 8) v += o;
  o = dpp_rows_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (lane & 16) v += o;
  o = dpp_rows_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  if (lane >= 32) v += o;
  return v;
}
// The previous lane's value (wave_shr:1); lane 0 reads 0.
__device__ __forceinline__ float wave_prev_f(float v) { return dpp_f<0x138>(v); }

template <typename E, bool SH>
__global__ __launch_bounds__(kAcceptDrawThreads) void k_accept_draw(VerifyParams p) {
  __shared__ AcceptDrawLds L;
  const int r = blockIdx.x;
  const int k = threadIdx.x;
  const int lane = k & (kWave - 1), wave = k / kWave;
  const int D = p.D;
  // Loads in two rounds: the request's scalars, thread k's token, its row
  // states and alpha partials (slots past a row's count are discarded
  // below); then p(d) and q(d).
  const int n = p.depth[r];
  const float T = p.temperature[r];
  const uint32_t rid = p.request_id ? p.request_id[r] : (uint32_t)r;
  const int64_t trow0 = p.target_row0[r];
  const int64_t drow0 = p.draft_row0 ? p.draft_row0[r] : 0;
  const int sync_err = *p.sync_error;
  if (k == 0) L.bits = 0u;

  // a team wait that expired is reported, not an error: the member took the
  // row normalisers from the full rows instead
  const uint32_t info = sync_err ? SV_BIT_SYNC_TIMEOUT : 0u;
  uint32_t bits = 0u;
  if (n < 0 || n > D) bits |= SV_BIT_BAD_DEPTH;
  if (!temperature_ok(T)) bits |= SV_BIT_BAD_TEMPERATURE;
  const bool live = (bits == 0u) && k <= n;
  const int64_t unit = (int64_t)r * (D + 1) + k;
  const bool pair = live && k < n;
  const bool greedy = T == 0.0f;
  // A row pair at T > 0 reads the row states its rates were taken against;
  // a single row (and every row at T = 0) merges its slot states.
  const bool pair_state = pair && !greedy;
  const int np_ = (live && !pair_state) ? p.S1 : 0;
  const int na_ = (pair_state && bits == 0u) ? p.pair_ns : 0;
  const int32_t tok_k = (k < D) ? p.tokens[(int64_t)r * D + k] : 0;
  float2 pv[kMergeChunk];
  float av[kMergeChunk];
  float2 pp = make_float2(-INFINITY, 0.0f), pq = make_float2(-INFINITY, 0.0f);
  if (k <= D) {
    const float2* prow_s = p.part_p + unit * p.S1;
    const float* arow_s = p.part_a + unit * p.S1;
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      pv[i] = prow_s[i];
      av[i] = arow_s[i];
    }
    pp = p.pair_p[unit];
    pq = p.pair_q[unit];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      if (i >= np_) pv[i] = make_float2(-INFINITY, greedy ? __int_as_float(INT32_MAX) : 0.0f);
      if (i >= na_) av[i] = 0.0f;
    }
  }
  int32_t d = 0;
  if (pair) {
    d = tok_k;
    if (d < 0 || (int64_t)d >= p.V) bits |= SV_BIT_BAD_TOKEN;
  }
  // p(d), q(d) for the accept test, issued before the merges
  float pd = 0.0f, qd = 0.0f;
  if (pair_state && bits == 0u && p.draft != nullptr) {
    pd = E::load1(row_view<E, SH>(p, false, trow0 + k).at(d), 0);
    qd = E::load1(row_view<E, SH>(p, true, drow0 + k).at(d), 0);
  }

  bool keep = true;
  float margin = INFINITY;
  float sl = 0.0f;
  SoftmaxPart sp{0.0f, 1.0f}, sq{0.0f, 1.0f};
  ArgMax am{0.0f, 0};
  if (live) {
    if (greedy) {
      am = merge_row_argmax(pv, p.part_p, unit, p.S1);
      if (!finite_f(am.v)) bits |= SV_BIT_BAD_ROW;
      if (k < n) keep = (d == am.i);
    } else {
      sl = kLog2e / T;
      sp = renormalise(pair_state ? SoftmaxPart{pp.x, pp.y}
                                  : merge_row(pv, p.part_p, unit, p.S1, np_, sl),
                       sl);
      if (!finite_f(sp.m)) bits |= SV_BIT_BAD_ROW;
      else if (!scale_ok(sp.m, sl)) bits |= SV_BIT_BAD_TEMPERATURE;
      if (k < n) {
        if (p.draft == nullptr) {
          bits |= SV_BIT_BAD_ROW;
        } else {
          sq = renormalise(SoftmaxPart{pq.x, pq.y}, sl);
          if (!finite_f(sq.m)) bits |= SV_BIT_BAD_ROW;
          else if (!scale_ok(sq.m, sl)) bits |= SV_BIT_BAD_TEMPERATURE;
        }
      }
      if (k < n && bits == 0u) {
        // log2 p(d) - log2 q(d), each as (x sl - R(m)) - log2 z: against
        // the same rounded reference as the row's sum z
        const float lp = __builtin_fmaf(pd, sl, -ref_of(sp.m, sl)) - __log2f(sp.z);
        const float lq = __builtin_fmaf(qd, sl, -ref_of(sq.m, sl)) - __log2f(sq.z);
        const float ratio = exp2_fast(lp - lq);
        const Philox4 w = philox4x32_10((uint32_t)k, rid, p.step, 0u, p.seed_lo, p.seed_hi);
        const float u = u24(w.w[0]);
        keep = u < ratio;  // false when ratio is NaN (p(d) = q(d) = 0)
        margin = fabsf(u - ratio);
      }
    }
  }
  __syncthreads();  // L.bits cleared
  if (bits) atomicOr(&L.bits, bits);
  __syncthreads();
  const uint32_t all_bits = L.bits;

  if (all_bits != 0u) {  // nothing emitted for an invalid request
    if (k <= D) p.out_tokens[(int64_t)r * (D + 1) + k] = -1;
    if (k < D && p.alpha) p.alpha[(int64_t)r * D + k] = 0.0f;
    if (k == 0) {
      p.accepted_len[r] = 0;
      p.num_out[r] = 0;
      if (p.diag) p.diag[r] = sv_diag{INFINITY, INFINITY, all_bits | info, 0};
    }
    return;
  }

  // First rejection: ballot of rejected positions in wavefront 0 (n <= 64).
  if (k < kWave) {
    const uint64_t rejected = __ballot(k < n && !keep);
    if (k == 0) L.tau = rejected ? (int)__builtin_ctzll(rejected) : n;
  }
  if (k <= kWave) L.margin[k] = (k < n) ? margin : INFINITY;
  __syncthreads();
  const int tau = L.tau;

  if (k <= D) {
    int32_t tok = -1;
    if (k < tau) tok = tok_k;
    else if (k == tau && T == 0.0f) tok = am.i;
    p.out_tokens[(int64_t)r * (D + 1) + k] = tok;
  }
  if (k < D && p.alpha) {
    float a = 0.0f;
    if (k < n) {
      if (T == 0.0f) {
        a = keep ? 1.0f : 0.0f;
      } else {
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) a += av[i];
        const float* pa = p.part_a + unit * p.S1;
        for (int j0 = kMergeChunk; j0 < p.pair_ns; j0 += kMergeChunk) {
          float v[kMergeChunk];
#pragma unroll
          for (int i = 0; i < kMergeChunk; ++i) v[i] = (j0 + i < p.pair_ns) ? pa[j0 + i] : 0.0f;
#pragma unroll
          for (int i = 0; i < kMergeChunk; ++i) a += v[i];
        }
      }
    }
    p.alpha[(int64_t)r * D + k] = a;
  }
  if (k == tau) {
    DrawState st;
    st.tau = tau;
    if (T == 0.0f) {
      st.mode = kDrawNone;
    } else {
      st.mode = (tau < n) ? kDrawResidual : kDrawBonus;
      st.prow = trow0 + tau;
      st.qrow = (tau < n) ? drow0 + tau : -1;
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
    L.st = st;
  }
  if (k == 0) {
    p.accepted_len[r] = tau;
    p.num_out[r] = tau + 1;
    if (p.diag) {
      float mm = INFINITY;
      for (int j = 0; j <= tau && j < n; ++j) mm = fminf(mm, L.margin[j]);
      p.diag[r] = sv_diag{mm, INFINITY, info, 0};
    }
  }
  __syncthreads();
  const DrawState st = L.st;
  if (st.mode == kDrawNone) return;  // workgroup-uniform

  // ---- draw: locate the slice holding t = u R (wavefront 0) ----
  const bool residual = st.mode == kDrawResidual;
  const int ns = residual ? p.pair_ns : p.single_ns;
  const int64_t slen = residual ? p.pair_len : p.single_len;
  const bool force64 = (p.flags & SV_FLAG_FORCE_FP64_DRAW) != 0u;
  const float cp = ref_of(st.mp, st.sl);
  if (wave == 0) {
    const int64_t dunit = (int64_t)r * (D + 1) + st.tau;
    float w = 0.0f;
    if (lane < ns) {
      const float2 ms = p.part_p[dunit * p.S1 + lane];
      const float a = residual ? p.part_a[dunit * p.S1 + lane] : 0.0f;
      const float ps = (ms.x == -INFINITY)
                           ? 0.0f
                           : ms.y * exp2_fast((ref_of(ms.x, st.sl) - cp) - st.lzp);
      w = residual ? fmaxf(ps - a, 0.0f) : ps;
    }
    // inclusive scan over the slices (fixed order)
    const float c = wave_scan_f(w);
    const float R = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(c), ns > 0 ? ns - 1 : 0));
    const float t = st.u * R;
    const uint64_t cross = __ballot(lane < ns && w > 0.0f && c > t);
    const int j = cross ? (int)__builtin_ctzll(cross) : -1;
    const float before = wave_prev_f(c);
    if (lane == 0) {
      L.slice = force64 ? -1 : j;
      L.t = t;
    }
    if (j >= 0 && lane == j) L.c0 = before;
  }
  __syncthreads();
  const int j = L.slice;
  bool found = false;
  int32_t y_hit = -1;
  float before_hit = 0.0f, at_hit = 0.0f;
  if (j >= 0) {
    // ---- scan inside slice j, kScanSpans spans of kChunk elements per round ----
    Weights32<E, SH> wt = weights32<E, SH>(p, st);
    const float t = L.t;
    float carry = L.c0;
    const int64_t lo = (int64_t)j * slen;
    const int64_t hi = min(p.V, lo + slen);
    // Thread k takes kPer elements of each span.  Span g is scanned as a
    // round of its own would be (wave totals in order, then the carry of the
    // spans before it), so the cumulative masses and the first crossing are
    // those of single-span rounds one after another; the spans share the
    // loads' latency and the round's two barriers.  Each round's raw logits
    // are loaded one round ahead, and the barriers order LDS only, so those
    // loads stay in flight while this round is scanned.
    constexpr int64_t kRound = (int64_t)kScanSpans * kChunk;
    Raw8<E> cur[kScanSpans], nxt[kScanSpans];
#pragma unroll
    for (int g = 0; g < kScanSpans; ++g) {
      const int64_t i0 = lo + g * kChunk + (int64_t)k * kPer;
      if (i0 < hi) load_raw8<E, SH>(wt.prow, wt.qrow, wt.has_q, i0, hi, cur[g]);
    }
    int buf = 0;
    for (int64_t base = lo; base < hi; base += kRound, buf ^= 1) {
#pragma unroll
      for (int g = 0; g < kScanSpans; ++g) {
        const int64_t i0 = base + g * kChunk + (int64_t)k * kPer;
        if (i0 + kRound < hi)
          load_raw8<E, SH>(wt.prow, wt.qrow, wt.has_q, i0 + kRound, hi, nxt[g]);
      }
      float w[kScanSpans][kPer], prev[kScanSpans];
#pragma unroll
      for (int g = 0; g < kScanSpans; ++g) {
        const int64_t i0 = base + g * kChunk + (int64_t)k * kPer;
        if (i0 < hi) {
          float a[kPer], b[kPer];
          unpack_raw8<E, SH>(cur[g], wt.prow, wt.qrow, wt.has_q, i0, hi, a, b);
          wt.from(a, b, w[g]);
        } else {
#pragma unroll
          for (int e = 0; e < kPer; ++e) w[g][e] = 0.0f;
        }
        cur[g] = nxt[g];
        float run = 0.0f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) run += w[g][e];
        // block exclusive scan of the thread sums (wavefront scans, wave
        // totals in order)
        const float incl = wave_scan_f(run);
        prev[g] = wave_prev_f(incl);
        if (lane == kWave - 1) L.wtot[buf][g][wave] = incl;
      }
      lds_barrier();
      float gcarry = carry;
#pragma unroll
      for (int g = 0; g < kScanSpans; ++g) {
        const int64_t i0 = base + g * kChunk + (int64_t)k * kPer;
        float wbase = 0.0f, total = 0.0f;
        for (int v = 0; v < kAcceptDrawWaves; ++v) {
          const float x = L.wtot[buf][g][v];
          if (v < wave) wbase += x;
          total += x;
        }
        const float excl = gcarry + (wbase + prev[g]);
        // the first element of this thread whose cumulative mass passes t
        float cum = excl;
        int first = -1;
        float bprev = 0.0f, bat = 0.0f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const float before = cum;
          cum += w[g][e];
          if (first < 0 && w[g][e] > 0.0f && cum > t) {
            first = e;
            bprev = before;
            bat = cum;
          }
        }
        const uint64_t hit = __ballot(first >= 0);
        const int fl = hit ? (int)__builtin_ctzll(hit) : -1;
        if (lane == 0) L.wfirst[buf][g][wave] = fl;
        if (lane == fl) {
          L.wy[buf][g][wave] = (int32_t)(i0 + first);
          L.wbefore[buf][g][wave] = bprev;
          L.wat[buf][g][wave] = bat;
        }
        gcarry += total;
      }
      lds_barrier();
      // the first span with a crossing, and in it the first wavefront
#pragma unroll
      for (int g = 0; g < kScanSpans; ++g) {
        if (found) break;
        for (int v = 0; v < kAcceptDrawWaves; ++v)
          if (L.wfirst[buf][g][v] >= 0) {
            found = true;
            y_hit = L.wy[buf][g][v];
            before_hit = L.wbefore[buf][g][v];
            at_hit = L.wat[buf][g][v];
            break;
          }
      }
      if (found) break;  // uniform
      carry = gcarry;
    }
  }
  if (k == 0) {
    float m = 0.0f;
    if (found) m = fminf(L.t - before_hit, at_hit - L.t);
    if (found && m >= kDrawMargin32) {
      p.out_tokens[(int64_t)r * (D + 1) + st.tau] = y_hit;
      if (p.diag) p.diag[r].draw_margin = m;
    } else {
      const bool residual = st.mode == kDrawResidual;
      DrawJob jb;
      jb.prow = st.prow;
      jb.qrow = residual ? st.qrow : 0;
      jb.invT = 1.0 / (double)st.T;
      jb.rho_e = residual ? exp2(log2_ratio_exact(st)) : 0.0;
      jb.mp = st.mp;
      jb.mq = st.mq;
      jb.u = st.u;
      jb.mode = st.mode;
      jb.r = r;
      jb.tau = st.tau;
      jb.y32 = found ? y_hit : -1;
      jb.pad = 0;
      p.fb_jobs[atomicAdd(p.fb_count, 1)] = jb;
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch sequence.
static void mark(const VerifyParams& p, int i, hipStream_t stream) {
  if (p.events && p.events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(p.events[i]), stream);
}

template <typename E>
static hipError_t launch_all(VerifyParams& p, int grid, hipStream_t stream) {
  // Team row pass when a row fits a team of at most 64 members and the team
  // kernel fits one workgroup per CU; otherwise the streaming row pass.
  // Vocabulary shards need the team pass (its members resolve the shard of
  // each vector).
  int32_t T = 0, nv = 0, slice = 0;
  const bool sharded = p.nshard > 1;
  const bool team = (p.flags & SV_FLAG_STREAMING_ROW_PASS) == 0u && grid <= kMaxTeamGrid &&
                    team_geometry(p.dtype, p.V, grid, &T, &nv, &slice);
  if (sharded && !team) return hipErrorInvalidValue;
  if (team) {
    p.S1 = T;
    p.team = T;
    p.nteams = grid / T;
    p.team_len = slice;
    // every row is cut into the team's slices
    p.pair_ns = p.single_ns = T;
    p.pair_len = p.single_len = slice;
  } else {
    p.team = 0;
    p.nteams = 0;
    // a row pair is one slice; single rows are cut into S1 segments
    p.pair_ns = 1;
    p.pair_len = p.V;
    p.single_ns = p.S1;
    p.single_len = p.seg1;
  }
  mark(p, 0, stream);
  launch_plan(p, stream);
  mark(p, 1, stream);
  bool done = false;
  if (team) done = launch_rowteam(p, grid, nv, stream) == hipSuccess;
  if (!done && sharded) return hipErrorInvalidValue;
  if (!done) {
    (void)hipGetLastError();
    if (team) {  // fall back: streaming pass with its own slot layout
      stats_geometry(p.B, p.D, p.V, &p.S1, &p.seg1);
      p.team = 0;
      p.nteams = 0;
      p.pair_ns = 1;
      p.pair_len = p.V;
      p.single_ns = p.S1;
      p.single_len = p.seg1;
    }
    launch_rowpass(p, grid, stream);
  }
  mark(p, 2, stream);
  if (sharded)
    hipLaunchKernelGGL((k_accept_draw<E, true>), dim3((unsigned)p.B), dim3(kAcceptDrawThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((k_accept_draw<E, false>), dim3((unsigned)p.B), dim3(kAcceptDrawThreads), 0,
                       stream, p);
  mark(p, 3, stream);
  launch_draw(p, grid, stream);
  mark(p, 4, stream);
  return hipGetLastError();
}

hipError_t launch_verify(VerifyParams& p, int grid, hipStream_t stream) {
  return (p.dtype == SV_DTYPE_BF16) ? launch_all<Bf16>(p, grid, stream)
                                    : launch_all<F32>(p, grid, stream);
}

}  // namespace sv
