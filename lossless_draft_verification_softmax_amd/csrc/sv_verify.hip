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
//   k_plan,      row statistics and acceptance rates (sv_rowpass.hip): the
//   k_rowpass    HBM-streaming pass.
//   k_accept     one workgroup per request: merge the segments, Philox accept
//                test per position, wavefront ballot + first set bit = tau,
//                emitted drafts, alpha, the draw's normalisers.
//   k_draw_*     inverse-CDF draw of the correction / bonus token
//                (sv_draw.hip).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
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
// k_accept: one workgroup (2 wavefronts) per request.  Thread k handles
// target row k (k <= n) and, for k < n, draft row k and the accept test.
template <typename E, bool SH>
__global__ __launch_bounds__(128) void k_accept(VerifyParams p) {
  using S = typename E::Storage;
  __shared__ uint32_t s_bits;
  __shared__ int s_tau;
  __shared__ float s_margin[128];
  const int r = blockIdx.x;
  const int k = threadIdx.x;
  const int D = p.D;
  // Loads in two rounds: the request's scalars, thread k's token and the
  // first chunk of its row states and alpha partials (read whatever the depth
  // and temperature turn out to be: the slots lie inside the workspace, and
  // those past a row's count are discarded below); then p(d) and q(d).
  const int n = p.depth[r];
  const float T = p.temperature[r];
  const uint32_t rid = p.request_id ? p.request_id[r] : (uint32_t)r;
  const int64_t trow0 = p.target_row0[r];
  const int64_t drow0 = p.draft_row0 ? p.draft_row0[r] : 0;
  const int sync_err = *p.sync_error;
  if (k == 0) s_bits = 0u;
  if (r == 0 && k == 0) *p.fb_count = 0;  // float64 draw queue, filled by k_draw_pick32

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
  // slots merged per row: every slot at T = 0 and for a single row, the
  // pair's slots for a row pair; q only for a T > 0 pair with draft logits
  const int np_ = live ? ((greedy || !pair) ? p.S1 : p.pair_slots) : 0;
  const int nq_ = (pair && !greedy && p.draft != nullptr) ? p.pair_slots : 0;
  const int na_ = (k < D && k < n && !greedy && bits == 0u && p.alpha) ? p.alpha_slots : 0;
  const int32_t tok_k = (k < D) ? p.tokens[(int64_t)r * D + k] : 0;
  float2 pv[kMergeChunk], qv[kMergeChunk];
  float av[kMergeChunk];
  {
    const float2* prow_s = p.part_p + unit * p.S1;
    const float2* qrow_s = p.part_q + unit * p.S1;
    const float* arow_s = p.part_a + unit * p.S1;
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      pv[i] = prow_s[i];
      qv[i] = qrow_s[i];
      av[i] = arow_s[i];
    }
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      if (i >= np_) pv[i] = make_float2(-INFINITY, greedy ? __int_as_float(INT32_MAX) : 0.0f);
      if (i >= nq_) qv[i] = make_float2(-INFINITY, 0.0f);
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
  if (pair && !greedy && bits == 0u && p.draft != nullptr) {
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
      sp = renormalise(merge_row(pv, p.part_p, unit, p.S1, np_, sl), sl);
      if (!finite_f(sp.m)) bits |= SV_BIT_BAD_ROW;
      if (k < n) {
        if (p.draft == nullptr) {
          bits |= SV_BIT_BAD_ROW;
        } else {
          sq = renormalise(merge_row(qv, p.part_q, unit, p.S1, nq_, sl), sl);
          if (!finite_f(sq.m)) bits |= SV_BIT_BAD_ROW;
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
  __syncthreads();  // s_bits cleared
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
      if (p.diag) p.diag[r] = sv_diag{INFINITY, INFINITY, all_bits | info, 0};
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
        for (int j0 = kMergeChunk; j0 < p.alpha_slots; j0 += kMergeChunk) {
          float v[kMergeChunk];
#pragma unroll
          for (int i = 0; i < kMergeChunk; ++i) v[i] = (j0 + i < p.alpha_slots) ? pa[j0 + i] : 0.0f;
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
    st.bits = 0u;
    st.need64 = 0;
    st.margin = INFINITY;
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
    p.req[r] = st;
  }
  if (k == 0) {
    p.accepted_len[r] = tau;
    p.num_out[r] = tau + 1;
    if (p.diag) {
      float mm = INFINITY;
      for (int j = 0; j <= tau && j < n; ++j) mm = fminf(mm, s_margin[j]);
      p.diag[r] = sv_diag{mm, INFINITY, info, 0};
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
    // with acceptance rates the team pass stores a pair's row states in slot 0
    p.pair_slots = p.alpha ? 1 : T;
    p.alpha_slots = T;
    p.team = T;
    p.nteams = grid / T;
    p.team_len = slice;
  } else {
    p.pair_slots = 1;
    p.alpha_slots = 1;
    p.team = 0;
    p.nteams = 0;
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
      p.pair_slots = 1;
      p.alpha_slots = 1;
    }
    launch_rowpass(p, grid, stream);
  }
  mark(p, 2, stream);
  if (sharded)
    hipLaunchKernelGGL((k_accept<E, true>), dim3((unsigned)p.B), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL((k_accept<E, false>), dim3((unsigned)p.B), dim3(128), 0, stream, p);
  mark(p, 3, stream);
  launch_draw(p, stream);
  mark(p, 4, stream);
  return hipGetLastError();
}

hipError_t launch_verify(VerifyParams& p, int grid, hipStream_t stream) {
  return (p.dtype == SV_DTYPE_BF16) ? launch_all<Bf16>(p, grid, stream)
                                    : launch_all<F32>(p, grid, stream);
}

}  // namespace sv
