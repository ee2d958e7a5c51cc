// sv_rowteam.hip -- the row pass with each row pair read from HBM once.
//
// Per T > 0 draft position the statistics pass needs both rows' softmax
// normalisers and then, with the full-row normalisers, sum_y min(p, q)
// (equation L_e2e of "AngelSpec: specialize the drafter...", section "MTP";
// one target pass over all drafts, "Tencent open-sources AngelSpec", section
// "Why one universal drafter underperforms").  The second sum needs the first
// pass finished over the whole row, so a row pair is split across a team of
// T workgroups (one per CU, all resident at once): each member keeps its
// slice of the pair in registers, computes
// the slice's (max, sum) for both rows, publishes them, and once the whole
// team has published computes its slice of sum min(p, q) from the same
// registers.  Nothing is read twice from memory.
//
// Each member walks a sequence of units: its team's row pairs, then its
// team's single rows (bonus rows at T > 0 and all target rows at T = 0) two
// at a time (one at a time in the vocabulary-sharded instantiation, whose
// registers are taken by per-thread shard addresses), always its own slice
// of the row.  A unit of two single rows holds the second one in the draft
// buffer; each row keeps its own temperature and kind (arg max at T = 0) and
// its own partial slot.
//
// Workgroup layout: waves 0..14 are data waves, wave 15 is the communication
// wave.  The data waves load rows and reduce them to per-wave states in LDS;
// the communication wave combines those states, writes the partial slots,
// publishes a row pair to the team, waits for the team and hands the row
// normalisers back through LDS.  For fp32 rows the last data wave to finish
// a pair's first pass combines and publishes it instead, before the step's
// barrier, so that the communication wave's polls queue behind no stores of
// its own (bf16 rows keep the communication wave: there a data wave's stores
// queue behind its row loads).  Loads complete in order per wave, so any
// wave that waited on a fresh global load (a poll) would also wait for all
// of its earlier row loads; keeping polls out of the data waves keeps their
// prefetches in flight.  For the same reason every data wave issues exactly
// the same loads on every path (lanes and units without data read a line of
// -inf), which lets the compiler wait on the oldest unit only.
//
// Software pipeline, step s: the data waves issue the loads of unit s + 2,
// take the first pass of unit s and then the second pass of unit s - 1.  The
// first pass of a row pair keeps its exponentials 2^(x sl - R(m_t)) (m_t
// the thread's maximum over its vectors) and parks them in LDS (one slot of
// 2 * NV * VEC float32 values per data thread, VEC elements per 16-byte
// vector; each thread reads back only what it wrote), so the second pass
// sums min(ep Kp, eq Kq) with one Kp = 2^(R(m_t) - c_p - lz_p) per thread
// and row (c_p + lz_p the log2 of the row's sum of 2^(x sl), lz_p small)
// instead of an exponential per element.  The communication wave gathers the
// team normalisers of unit s in the same step.  Three register buffers
// rotate (unit s and two units in flight).
//
// Team exchange: member m publishes its slice states of its n-th row pair as
// four 64-bit words (value bits | (n + 1) << 32) in ring slot n mod 4; a
// reader accepts a word only if its tag is n + 1, so no fences are needed.
// A member publishes n after its barrier n - 1 (at the end of its data step
// n, or after barrier n from the communication wave), so after its
// communication wave has read every member's n - 2; each of those was
// published after that member's barrier n - 3, by when that member had read
// n - 4, the previous user of the ring slot.  The words
// are cleared before each launch.  The wait is bounded.  A team needs all of
// its members resident at once, which holds when the kernel has the device to
// itself (one workgroup per CU); when other work holds CUs a member may not
// start until others finish.  So a member whose wait expires does not depend
// on the team any more: its communication wave streams the pair's two full
// rows itself and takes their states from them (slower, same results to
// rounding), sets a word that the accept kernel reports as
// SV_BIT_SYNC_TIMEOUT, and from then on polls each later pair once before
// doing the same.  Tags keep this sound when members fall out of step: a
// record is used only if it carries the pair's own ordinal.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "specverify.h"
#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_shard.hpp"

namespace sv {

constexpr int kTeamThreads = 1024;
constexpr int kDataWaves = kTeamThreads / kWave - 1;
constexpr int kDataThreads = kDataWaves * kWave;
constexpr uint32_t kSpinLimit = 1u << 20;  // polls; a normal wait takes a few

template <int NV>
struct Regs {
  uint4 p[NV];
  uint4 q[NV];
};

// A unit of work, held in scalar registers.
struct UnitDesc {
  int64_t trow;     // target row index
  int64_t drow;     // draft row index (row pairs); second target row of a single unit, or -1
  uint32_t code;    // request << 7 | position
  float sl;         // log2(e) / T
  int32_t kind;     // 0 none, 1 row pair, 2 single row, 3 single row at T = 0
  int32_t ordinal;  // pair ordinal within the team
};

// The workgroup's slice of every row it works on: columns [lo, hi) of the
// full row, of which [lo, vhi) are nvec whole 16-byte vectors.  Column i
// lies at element i - toff of the buffers tgt / dft.  Without vocabulary
// shards these are the row buffers and toff = 0.  With shards the slices
// tile the concatenated row as they do an unsharded one and may cross a
// shard boundary; the shard width is a whole number of vectors, so each
// vector lies in one shard and each thread resolves its vectors' shard
// addresses once (LanePtrs).  tgt / dft are then the last shard's buffers,
// which hold the ragged tail (the columns past the last whole vector).
struct Slice {
  int64_t lo, vhi, hi, nvec, toff;
  const void* tgt;
  const void* dft;
};

template <typename E, bool SH>
__device__ __forceinline__ Slice make_slice(const VerifyParams& p, int member) {
  constexpr int VEC = E::kPerVec;
  Slice sc;
  sc.toff = 0;
  sc.tgt = p.target;
  sc.dft = p.draft;
  if constexpr (SH) {
    const int last = p.nshard - 1;
    sc.toff = (int64_t)last * p.shard_w;
    sc.tgt = p.shard_tab[last];
    sc.dft = p.shard_tab[kMaxShards + last];
  }
  sc.lo = (int64_t)member * p.team_len;
  sc.hi = min(p.V, sc.lo + (int64_t)p.team_len);
  if (sc.hi < sc.lo) sc.hi = sc.lo;
  sc.nvec = (sc.hi - sc.lo) / VEC;
  sc.vhi = sc.lo + sc.nvec * VEC;
  return sc;
}

// Sharded rows: the address in row 0 of each of this thread's NV vectors,
// in the target and in the draft shards.  Vectors past the slice get any
// address inside the table's range; they are never read.
template <int NV>
struct LanePtrs {
  const char* t[NV];
  const char* d[NV];
};

template <typename E, int NV>
__device__ __forceinline__ LanePtrs<NV> lane_ptrs(const VerifyParams& p, const Slice& sc) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  const int64_t wv = p.shard_w / VEC;  // vectors per shard
  LanePtrs<NV> lp;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t g = sc.lo / VEC + (int64_t)threadIdx.x + (int64_t)kDataThreads * i;
    const int s = (int)min(g / wv, (int64_t)(p.nshard - 1));
    const int64_t o = (g - (int64_t)s * wv) * VEC * (int64_t)sizeof(S);
    lp.t[i] = static_cast<const char*>(p.shard_tab[s]) + o;
    lp.d[i] = static_cast<const char*>(p.shard_tab[kMaxShards + s]) + o;
  }
  return lp;
}

// Shared state, double-buffered by unit parity (see the step order above).
struct TeamLds {
  SoftmaxPart sm[2][kDataWaves][2];  // per-wave (max, sum) of p and q
  ArgMax am[2][kDataWaves][2];       // per-wave arg max at T = 0, per single row
  float acc[2][kDataWaves];          // per-wave sum of min(p, q)
  float c[2][2];                     // team row values of p and q in log2:
  float lz[2][2];                    // a reference c and a small remainder lz
  float ep[2];                       // 2^-lz of the target row
  float rq[2];                       // 2^(lz_p - lz_q)
  int ok[2];
  int arrived[2];                    // data waves done with a row pair's first pass
};

// Work items are read-only here and uniform across the workgroup: read them
// through the constant address space, so that they become scalar loads that
// count against the scalar-memory counter rather than the in-order vector-load
// counter that tracks the rows in flight.
__device__ __forceinline__ void load_item(UnitDesc& u, const PlanItem* items, int64_t n) {
  const __attribute__((address_space(4))) PlanItem* c =
      (const __attribute__((address_space(4))) PlanItem*)items;
  u.trow = c[n].trow;
  u.drow = c[n].drow;
  u.code = c[n].code;
  u.sl = c[n].sl;
}

__device__ __forceinline__ UnitDesc no_unit() {
  UnitDesc u;
  u.trow = 0;
  u.drow = 0;
  u.code = 0u;
  u.sl = 0.0f;
  u.kind = 0;
  u.ordinal = 0;
  return u;
}

// Single rows per team member: the team's singles are items team,
// team + nteams, ...; single unit j holds the team's singles PS j .. PS j +
// PS - 1 (PS = 2, or 1 where the pairing's registers do not fit: the
// vocabulary-sharded instantiation).
__device__ __forceinline__ int64_t single_units(int64_t my_singles, int PS) {
  return (my_singles + PS - 1) / PS;
}

__device__ __forceinline__ int64_t team_single(const VerifyParams& p, int team, int64_t m) {
  return (int64_t)team + (int64_t)p.nteams * m;
}

// Unit j of this workgroup: its team's row pairs (items team, team + nteams,
// ...) and then its team's single rows (dealt the same way), two per unit;
// the workgroup always takes slice `member` of the row.
__device__ __forceinline__ UnitDesc unit_at(const VerifyParams& p, int64_t j, int64_t n,
                                            int team, int64_t my_pairs, int64_t my_singles,
                                            int PS) {
  if (j >= n) return no_unit();
  UnitDesc u;
  if (j < my_pairs) {
    load_item(u, p.plan_pairs, (int64_t)team + (int64_t)p.nteams * j);
    u.kind = 1;
    u.ordinal = (int32_t)j;
  } else {
    const int64_t m = PS * (j - my_pairs);
    const int64_t it = team_single(p, team, m);
    load_item(u, p.plan_singles, it);
    const __attribute__((address_space(4))) PlanItem* c =
        (const __attribute__((address_space(4))) PlanItem*)p.plan_singles;
    u.kind = (c[it].T == 0.0f) ? 3 : 2;
    u.drow = (PS == 2 && m + 1 < my_singles) ? c[it + p.nteams].trow : -1;
    u.ordinal = 0;
  }
  return u;
}

// Every row pair gets its sum of min(p, q) per slice (the acceptance rate
// and, per slice, the draw's residual masses), whether or not the caller
// asked for the rates.
__device__ __forceinline__ bool wants_alpha(const VerifyParams& p, const UnitDesc& u) {
  (void)p;
  return u.kind == 1;
}

__device__ __forceinline__ int64_t unit_slot(const VerifyParams& p, const UnitDesc& u,
                                             int member) {
  const int64_t unit = (int64_t)(u.code >> 7) * (p.D + 1) + (u.code & 127u);
  return unit * p.S1 + member;
}

// A 16-byte line of -inf elements (bf16, fp32): the loads of lanes without
// data read it, so their values drop out of every max and sum unmasked.  It
// is never written; it is not declared const so that it lives in the global
// address space like the rows and the loads stay global loads.
__device__ uint4 kNegInfLine[2] = {{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u},
                                         {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u}};

template <typename E>
__device__ __forceinline__ const uint4* neg_inf_line() {
  return &kNegInfLine[E::kPerVec == 8 ? 0 : 1];
}

// Issues the 2 * NV loads of a unit: the target and draft rows of a pair,
// or the two target rows of a single unit.  Vectors outside the slice, the
// absent second row of a single unit and every vector of an empty unit read
// the -inf line instead.
template <typename E, int NV, bool SH, int PS>
__device__ __forceinline__ void load_unit(const VerifyParams& p, const UnitDesc& u,
                                          const Slice& sc, const LanePtrs<NV>& lp, Regs<NV>& R,
                                          const uint4* dummy) {
  using S = typename E::Storage;
  constexpr int VEC = E::kPerVec;
  const int64_t nvec = u.kind == 0 ? 0 : sc.nvec;
  const bool pair = u.kind == 1;
  const bool second = pair || (PS == 2 && u.drow >= 0);
  if constexpr (SH) {
    const int64_t tb = u.trow * p.stride * (int64_t)sizeof(S);
    const int64_t db = u.drow * p.stride * (int64_t)sizeof(S);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t v = (int64_t)threadIdx.x + (int64_t)kDataThreads * i;
      const bool in = v < nvec;
      const void* pa = in ? (const void*)(lp.t[i] + tb) : (const void*)dummy;
      const char* qbase = (PS == 2 && !pair) ? lp.t[i] : lp.d[i];
      const void* qa = (in && second) ? (const void*)(qbase + db) : (const void*)dummy;
      R.p[i] = load16(pa);
      R.q[i] = load16(qa);
    }
  } else {
    const S* prow = row_ptr<E>(sc.tgt, u.trow, p.stride) + sc.lo;
    const S* qrow = row_ptr<E>((PS == 2 && !pair) ? sc.tgt : sc.dft, u.drow, p.stride) + sc.lo;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t v = (int64_t)threadIdx.x + (int64_t)kDataThreads * i;
      const bool in = v < nvec;
      const void* pa = in ? (const void*)(prow + v * VEC) : (const void*)dummy;
      const void* qa = (in && second) ? (const void*)(qrow + v * VEC) : (const void*)dummy;
      R.p[i] = load16(pa);
      R.q[i] = load16(qa);
    }
  }
}


// ---------------------------------------------------------------------------
// Data waves.

// (max, sum) of N values with their exponentials kept: e[i] = 2^(x[i] sl -
// msl), msl = R(m) (m = 0 if every value is -inf), summed in the order of
// softmax_group from an empty state.
template <int N>
__device__ __forceinline__ SoftmaxPart softmax_keep(const float (&x)[N], float sl, float (&e)[N],
                                                    float& msl) {
  float cm = x[0];
#pragma unroll
  for (int i = 1; i + 1 < N; i += 2) cm = vmax3(cm, x[i], x[i + 1]);
  if constexpr ((N % 2) == 0) cm = vmax(cm, x[N - 1]);
  const float ms = (cm == -INFINITY) ? 0.0f : cm;
  msl = ref_of(ms, sl);
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = exp2_fast(__builtin_fmaf(x[i], sl, -msl));
  constexpr int C = N % 8 == 0 ? 8 : (N < 8 ? N : 4);
  static_assert(N % C == 0, "group size must be a multiple of the chunk");
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < N; c += C) {
    float t[C];
#pragma unroll
    for (int i = 0; i < C; ++i) t[i] = e[c + i];
#pragma unroll
    for (int w = 1; w < C; w <<= 1) {
#pragma unroll
      for (int i = 0; i + w < C; i += 2 * w) t[i] += t[i + w];
    }
    acc = (c == 0) ? t[0] : acc + t[0];
  }
  return {cm, acc};
}

// Arg max of a wave's share of a bf16 row slice held in V, by integer keys:
// an element's key is its 16 bits mapped to unsigned order (the sign bit
// flipped for a positive value, every bit for a negative one) above 15 minus
// its position among the thread's 8 NV elements, so that the unsigned
// maximum of a thread's keys is its largest value at its first position;
// the lane and the vector index then join the position, and one 32-bit
// maximum over the wave gives the wave's first maximal column.  Returns
// false when the float path must decide: a maximum of zero (-0 and +0 tie
// as values) or a slice with a ragged tail.  A NaN anywhere in the wave's
// share gives the state (NaN, none), an all -inf share (-inf, none).
template <int NV>
__device__ __forceinline__ bool bf16_argmax_keys(const uint4 (&V)[NV], const Slice& sc, ArgMax& out) {
  typedef short short2v __attribute__((ext_vector_type(2)));
  static_assert(NV <= 2, "positions must fit 4 key bits");
  if (sc.vhi < sc.hi) return false;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t d[4] = {V[i].x, V[i].y, V[i].z, V[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // 0xffff in each half holding a negative value
      const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(short2v, d[k]) >> (short)15);
      const uint32_t o = d[k] ^ (neg | 0x80008000u);
      const uint32_t klo = (o << 16) | (uint32_t)(15 - (8 * i + 2 * k));
      const uint32_t khi = (o & 0xFFFF0000u) | (uint32_t)(14 - (8 * i + 2 * k));
      kmax = max(max(kmax, klo), khi);
      kmin = min(min(kmin, klo), khi);
    }
  }
  // NaN: above +inf (0xff80 maps to 0xff80) or below -inf (0x007f)
  const bool nan = __ballot(kmax >= 0xFF810000u || kmin < 0x007F0000u) != 0ull;
  const uint32_t local = 15u - (kmax & 15u);  // vector * 8 + element
  // the lane, taken here rather than kept live across the row loop
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const uint32_t rank = ((local >> 3) << 9) | (lane << 3) | (local & 7u);
  const uint32_t wk = (uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(wave_allreduce(
      __uint_as_float((kmax & 0xFFFF0000u) | (0xFFFFu - rank)),
      [](float a, float b) { return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b))); })));
  const uint32_t ord = wk >> 16;
  if (nan) {
    out = ArgMax{__int_as_float(0x7fc00000), INT32_MAX};
    return true;
  }
  if (ord == 0x8000u) return false;  // +0
  if (ord == 0x007Fu) {  // -inf
    out = ArgMax{-INFINITY, INT32_MAX};
    return true;
  }
  const uint32_t bits = ord >= 0x8000u ? (ord ^ 0x8000u) : (ord ^ 0xFFFFu);
  const uint32_t r = 0xFFFFu - (wk & 0xFFFFu);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t v = (int64_t)(wave * kWave + (int)((r >> 3) & 63u)) + (int64_t)kDataThreads * (r >> 9);
  out = ArgMax{__uint_as_float(bits << 16), (int32_t)(sc.lo + v * 8 + (r & 7u))};
  return true;
}

// First pass of one single row (a target row) held in V: the slice arg max
// at T = 0 (kind 3), else the slice (max, sum) with log2(e)/T = sl; one
// state per wave into LDS entry `slot` (0 or 1) of the unit's states.
template <typename E, int NV>
__device__ __forceinline__ void single_first(const VerifyParams& p, const Slice& sc,
                                             const uint4 (&V)[NV], int64_t trow, int kind,
                                             float sl, TeamLds& L, int b, int slot,
                                             float (&e)[2 * NV * E::kPerVec]) {
  constexpr int VEC = E::kPerVec;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t lo = sc.lo, vhi = sc.vhi, hi = sc.hi;
  const auto* prow = row_ptr<E>(sc.tgt, trow, p.stride);
  if (kind == 3) {
    if constexpr (E::kPerVec == 8) {
      ArgMax w;
      if (bf16_argmax_keys<NV>(V, sc, w)) {
        if (lane == 0) L.am[b][wave][slot] = w;
        return;
      }
    }
    // arg max of this thread's vectors: the maximum (NaN propagates), then
    // its first position by a compare-select walk from the last element; a
    // maximum of -inf or NaN has no position
    float xs[NV][VEC];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      E::unpack(V[i], xs[i]);
#pragma unroll
      for (int j = 0; j < VEC; ++j) mx = vmax(mx, xs[i][j]);
    }
    ArgMax a{mx, INT32_MAX};
    if (mx > -INFINITY) {
      const int32_t base = (int32_t)(lo + (int64_t)threadIdx.x * VEC);
#pragma unroll
      for (int i = NV - 1; i >= 0; --i)
#pragma unroll
        for (int j = VEC - 1; j >= 0; --j)
          if (xs[i][j] == mx) a.i = base + (kDataThreads * i * VEC + j);
    }
    for (int64_t i = vhi + threadIdx.x; i < hi; i += kDataThreads)
      a = argmax_merge(a, ArgMax{E::load1(prow, i - sc.toff), (int32_t)i});
    // wave merge: the largest value (a NaN in any lane wins, by ballot), then
    // the smallest position among the lanes holding it (-0 and +0 compare
    // equal, as in the per-element walk)
    const bool nan = __ballot(a.v != a.v) != 0ull;
    const float wm = wave_allreduce(a.v, [](float x, float y) { return fmaxf(x, y); });
    const int32_t wi = __float_as_int(wave_allreduce(
        __int_as_float(a.v == wm ? a.i : INT32_MAX),
        [](float x, float y) { return __int_as_float(min(__float_as_int(x), __float_as_int(y))); }));
    a = nan ? ArgMax{__int_as_float(0x7fc00000), INT32_MAX}
            : ArgMax{wm, wm == -INFINITY ? INT32_MAX : wi};
    if (lane == 0) L.am[b][wave][slot] = a;
    return;
  }
  float x[VEC * NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) E::unpack(V[i], *reinterpret_cast<float(*)[VEC]>(&x[i * VEC]));
  float msl;
  SoftmaxPart sp = softmax_keep<VEC * NV>(x, sl, *reinterpret_cast<float(*)[VEC * NV]>(&e[0]), msl);
  for (int64_t i = vhi + threadIdx.x; i < hi; i += kDataThreads) {
    float x1[1] = {E::load1(prow, i - sc.toff)};
    softmax_group<1>(sp, x1, sl);
  }
  sp = wave_merge_ref(sp, sl);
  if (lane == 0) L.sm[b][wave][slot] = sp;
}

// The member's slice state of row pair u from the data waves' states (a
// fixed reduction tree over the lanes; `sum` is reduced alongside), into its
// partial slots, and its publication to the team: four 64-bit words (value
// bits | (ordinal + 1) << 32) in ring slot ordinal mod 4.  Run by the
// communication wave after the step's barrier, or (kDataPublish) by the last
// data wave to finish the pair's first pass.
__device__ __forceinline__ void publish_pair(const VerifyParams& p, const UnitDesc& u,
                                             const TeamLds& L, int b, int team, int member,
                                             float& sum) {
  // The lane index is taken afresh here (mbcnt, in a volatile asm the
  // compiler cannot hoist): the data waves' registers are full, and a
  // long-lived copy would be spilled and its reload would wait for every row
  // load in flight.
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const float sl = u.sl;
  SoftmaxPart sp{-INFINITY, 0.0f}, sq{-INFINITY, 0.0f};
  if (lane < kDataWaves) {
    sp = L.sm[b][lane][0];
    sq = L.sm[b][lane][1];
  }
  wave_merge_ref2(sp, sq, true, sum, sl);
  const int64_t slot = unit_slot(p, u, member);
  if (lane == 0) {
    p.part_p[slot] = make_float2(sp.m, sp.z);
    p.part_q[slot] = make_float2(sq.m, sq.z);
  }
  if (lane < 4) {
    const float v = lane == 0 ? sp.m : lane == 1 ? sp.z : lane == 2 ? sq.m : sq.z;
    const uint64_t tag = (uint64_t)(uint32_t)(u.ordinal + 1) << 32;
    const int64_t rec = ((int64_t)team * 4 + (u.ordinal & 3)) * p.team + member;
    __hip_atomic_store(&p.team_xch[rec * 4 + lane], tag | (uint64_t)__float_as_uint(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// First pass of a unit over this thread's vectors: for a row pair the slice
// (max, sum) of p and q, keeping the exponentials; for a single unit each of
// its rows by single_first (the second row's temperature is read from its
// work item, item2).  One state per wave and row into LDS.
template <typename E, int NV, int PS>
__device__ __forceinline__ void first_pass_data(const VerifyParams& p, const UnitDesc& u,
                                                const Slice& sc, const Regs<NV>& R, TeamLds& L,
                                                int b, float (&e)[2 * NV * E::kPerVec],
                                                float& mslp, float& mslq, int64_t item2) {
  constexpr int VEC = E::kPerVec;
  if (u.kind == 0) return;
  if (u.kind != 1) {
    single_first<E, NV>(p, sc, R.p, u.trow, u.kind, u.sl, L, b, 0, e);
    if (PS == 2 && u.drow >= 0) {
      const __attribute__((address_space(4))) PlanItem* c =
          (const __attribute__((address_space(4))) PlanItem*)p.plan_singles;
      const float T2 = c[item2].T, sl2 = c[item2].sl;
      single_first<E, NV>(p, sc, R.q, u.drow, T2 == 0.0f ? 3 : 2, sl2, L, b, 1, e);
    }
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int64_t vhi = sc.vhi, hi = sc.hi;
  const auto* prow = row_ptr<E>(sc.tgt, u.trow, p.stride);
  const float sl = u.sl;
  float x[VEC * NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) E::unpack(R.p[i], *reinterpret_cast<float(*)[VEC]>(&x[i * VEC]));
  SoftmaxPart sp = softmax_keep<VEC * NV>(x, sl, *reinterpret_cast<float(*)[VEC * NV]>(&e[0]), mslp);
  for (int64_t i = vhi + threadIdx.x; i < hi; i += kDataThreads) {
    float x1[1] = {E::load1(prow, i - sc.toff)};
    softmax_group<1>(sp, x1, sl);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) E::unpack(R.q[i], *reinterpret_cast<float(*)[VEC]>(&x[i * VEC]));
  SoftmaxPart sq = softmax_keep<VEC * NV>(x, sl, *reinterpret_cast<float(*)[VEC * NV]>(&e[VEC * NV]), mslq);
  const auto* qrow = row_ptr<E>(sc.dft, u.drow, p.stride);
  for (int64_t i = vhi + threadIdx.x; i < hi; i += kDataThreads) {
    float x1[1] = {E::load1(qrow, i - sc.toff)};
    softmax_group<1>(sq, x1, sl);
  }
  sp = wave_merge_ref(sp, sl);
  sq = wave_merge_ref(sq, sl);
  if (lane == 0) {
    L.sm[b][wave][0] = sp;
    L.sm[b][wave][1] = sq;
  }
}

// After a row pair's first pass: the last data wave to arrive publishes the
// pair (the fetch-add orders every wave's states before it) and resets the
// counter, which is next used two steps later, after a barrier.
__device__ __forceinline__ void arrive_pair(const VerifyParams& p, const UnitDesc& u, TeamLds& L,
                                            int b, int team, int member) {
  const int lane = threadIdx.x & (kWave - 1);
  int order = 0;
  if (lane == 0)
    order = __hip_atomic_fetch_add(&L.arrived[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  order = __builtin_amdgcn_readfirstlane(order);
  if (order == kDataWaves - 1) {
    float none = 0.0f;
    publish_pair(p, u, L, b, team, member, none);
    if (lane == 0) L.arrived[b] = 0;
  }
}

// Second pass of a row pair: this thread's share of sum min(p, q) with the
// team's row values c + lz (log2 of each row's sum of 2^(x sl)), from the
// exponentials kept by the first pass: p = ep Kp and q = eq Kq with
// Kp = 2^(mslp - c_p) 2^-lz_p, Kq = 2^(mslq - c_q) 2^-lz_q, where mslp - c_p
// and mslq - c_q are exact integers (differences of integer references) and
// 2^-lz_p, 2^(lz_p - lz_q) are the row pair's two constants, so that
// Kp = ldexp(2^-lz_p, mslp - c_p) and Kq / Kp = ldexp(2^(lz_p - lz_q),
// (mslq - c_q) - (mslp - c_p)) are exact scalings of them; then
// min(p, q) = Kp min(ep, eq Kq / Kp).  Kp <= 2^(1/2) (the thread maximum is
// at most the row maximum, and R(m_t) at most half above m_t sl); a thread
// whose Kp is under 2^-60 holds p values that small and adds nothing.  One
// sum per wave into LDS.
template <typename E, int NV>
__device__ __forceinline__ void second_pass_data(const VerifyParams& p, const UnitDesc& u,
                                                 const Slice& sc,
                                                 const uint4 (&ex)[2 * NV * E::kPerVec / 4],
                                                 TeamLds& L, int b, float mslp, float mslq) {
  constexpr int VEC = E::kPerVec;
  constexpr int H = NV * VEC / 4;  // 16-byte vectors of one row's exponentials

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const float sl = u.sl;
  const float cp = L.c[b][0], cq = L.c[b][1];
  const float lzp = L.lz[b][0], lzq = L.lz[b][1];
  const bool ok = L.ok[b] != 0;
  float acc = 0.0f;
  if (ok) {
    const int ip = (int)(mslp - cp), iq = (int)(mslq - cq);
    const float kp = ip > -60 ? __builtin_ldexpf(L.ep[b], ip) : 0.0f;
    const float r = ip > -60 ? __builtin_ldexpf(L.rq[b], iq - ip) : 0.0f;
    // chunks of G 16-byte vectors of each row
    constexpr int G = H % 2 == 0 ? 2 : 1;
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < H; c += G) {
      float m[4 * G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // ep and eq r are non-negative floats, which order as their bit
        // patterns do: an integer minimum, with no canonicalisation of the
        // values read back from LDS
        const uint4 a = ex[c + h], q = ex[H + c + h];
        m[4 * h + 0] = __uint_as_float(min(a.x, __float_as_uint(__uint_as_float(q.x) * r)));
        m[4 * h + 1] = __uint_as_float(min(a.y, __float_as_uint(__uint_as_float(q.y) * r)));
        m[4 * h + 2] = __uint_as_float(min(a.z, __float_as_uint(__uint_as_float(q.z) * r)));
        m[4 * h + 3] = __uint_as_float(min(a.w, __float_as_uint(__uint_as_float(q.w) * r)));
      }
#pragma unroll
      for (int w = 1; w < 4 * G; w <<= 1) {
#pragma unroll
        for (int j = 0; j + w < 4 * G; j += 2 * w) m[j] += m[j + w];
      }
      sum += m[0];
    }
    acc = sum * kp;
    const auto* prow = row_ptr<E>(sc.tgt, u.trow, p.stride);
    const auto* qrow = row_ptr<E>(sc.dft, u.drow, p.stride);
    for (int64_t i = sc.vhi + threadIdx.x; i < sc.hi; i += kDataThreads)
      acc += exp2_fast(fminf(__builtin_fmaf(E::load1(prow, i - sc.toff), sl, -cp) - lzp,
                             __builtin_fmaf(E::load1(qrow, i - sc.toff), sl, -cq) - lzq));
  }
  acc = wave_sum(acc);
  if (lane == 0) L.acc[b][wave] = acc;
}

// ---------------------------------------------------------------------------
// Communication wave.

// The second row of a single unit, as the communication wave holds it.
struct SecondRow {
  uint32_t code;  // request << 7 | position
  float sl;       // log2(e) / T
  int32_t kind;   // 0 none, 2 single row, 3 single row at T = 0
};

__device__ __forceinline__ int64_t code_slot(const VerifyParams& p, uint32_t code, int member) {
  const int64_t unit = (int64_t)(code >> 7) * (p.D + 1) + (code & 127u);
  return unit * p.S1 + member;
}

// A single row's slice state from the data waves' states (entry `slot` of
// the unit's), into its partial slot; `sum` is reduced alongside.
__device__ __forceinline__ void comm_single_softmax(const VerifyParams& p, const TeamLds& L, int b,
                                                    int slot, float sl, int64_t dst, float& sum) {
  const int lane = threadIdx.x & (kWave - 1);
  SoftmaxPart sp{-INFINITY, 0.0f}, none{-INFINITY, 0.0f};
  if (lane < kDataWaves) sp = L.sm[b][lane][slot];
  wave_merge_ref2(sp, none, false, sum, sl);
  if (lane == 0) p.part_p[dst] = make_float2(sp.m, sp.z);
}

__device__ __forceinline__ void comm_single_argmax(const VerifyParams& p, const TeamLds& L, int b,
                                                   int slot, int64_t dst) {
  const int lane = threadIdx.x & (kWave - 1);
  ArgMax a = (lane < kDataWaves) ? L.am[b][lane][slot] : ArgMax{-INFINITY, INT32_MAX};
  for (int m = 1; m < kWave; m <<= 1) {
    ArgMax o{__shfl_xor(a.v, m), __shfl_xor(a.i, m)};
    a = argmax_merge(a, o);
  }
  if (lane == 0) p.part_p[dst] = make_float2(a.v, __int_as_float(a.i));
}

// Combines the data waves' first-pass states of a unit (a fixed reduction
// tree over the lanes) into the partial slots and publishes a row pair (DP:
// the last data wave has done that already), with the second-pass sums of
// unit ua reduced alongside.
template <bool DP>
__device__ __forceinline__ void first_pass_comm(const VerifyParams& p, const UnitDesc& u,
                                                const SecondRow& u2, const TeamLds& L, int b,
                                                int team, int member, const UnitDesc& ua, int ba) {
  const int lane = threadIdx.x & (kWave - 1);
  // the second-pass sums of unit ua are reduced alongside (same tree as
  // a lone wave sum)
  const bool fin = wants_alpha(p, ua);
  float acc = (fin && lane < kDataWaves) ? L.acc[ba][lane] : 0.0f;
  if (u.kind != 1) {
    // single unit (or none): its first row, with the second-pass sum of unit
    // ua reduced alongside a softmax row or alone, then its second row
    if (u.kind == 2) {
      comm_single_softmax(p, L, b, 0, u.sl, code_slot(p, u.code, member), acc);
    } else {
      if (fin) acc = wave_sum(acc);
      if (u.kind == 3) comm_single_argmax(p, L, b, 0, code_slot(p, u.code, member));
    }
    if (fin && lane == 0) p.part_a[unit_slot(p, ua, member)] = acc;
    if (u2.kind == 2) {
      float none = 0.0f;
      comm_single_softmax(p, L, b, 1, u2.sl, code_slot(p, u2.code, member), none);
    } else if (u2.kind == 3) {
      comm_single_argmax(p, L, b, 1, code_slot(p, u2.code, member));
    }
    return;
  }
  if constexpr (DP) {
    // a row pair: merged and published by the last data wave; only the
    // second-pass sums of unit ua remain
    if (fin) acc = wave_sum(acc);
  } else {
    publish_pair(p, u, L, b, team, member, acc);
  }
  if (fin && lane == 0) p.part_a[unit_slot(p, ua, member)] = acc;
}

// Loads of one member's exchange record (lane m < T reads member m's record
// of row pair u).
struct TeamPoll {
  uint64_t w[4];
};

__device__ __forceinline__ TeamPoll team_poll(const VerifyParams& p, const UnitDesc& u,
                                              int team) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t rec = ((int64_t)team * 4 + (u.ordinal & 3)) * p.team + lane;
  TeamPoll t;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    t.w[k] = (lane < p.team) ? __hip_atomic_load(&p.team_xch[rec * 4 + k], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : 0ull;
  return t;
}

// The state (max, sum) of one whole row, streamed by the communication wave
// alone: the fallback of a member whose team wait expired.  U 16-byte loads
// per lane in flight, then the ragged tail element by element; the exact wave
// merge at the end.
template <typename E, bool SH>
__device__ SoftmaxPart wave_row_state(const VerifyParams& p, bool draft, int64_t row, float sl) {
  constexpr int VEC = E::kPerVec;
  constexpr int U = SH ? 2 : 8;
  const int lane = threadIdx.x & (kWave - 1);
  const RowView<E, SH> rv = row_view<E, SH>(p, draft, row);
  const int64_t nvec = p.V / VEC;
  SoftmaxPart s{-INFINITY, 0.0f};
  int64_t v = lane;
  for (; v + (U - 1) * kWave < nvec; v += U * kWave) {
    uint4 raw[U];
#pragma unroll
    for (int i = 0; i < U; ++i) raw[i] = load16(rv.at((v + i * kWave) * VEC));
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float x[VEC];
      E::unpack(raw[i], x);
      softmax_group<VEC>(s, x, sl);
    }
  }
  for (; v < nvec; v += kWave) {
    float x[VEC];
    E::unpack(load16(rv.at(v * VEC)), x);
    softmax_group<VEC>(s, x, sl);
  }
  for (int64_t i = nvec * VEC + lane; i < p.V; i += kWave) {
    float x1[1] = {E::load1(rv.at(i), 0)};
    softmax_group<1>(s, x1, sl);
  }
  return wave_merge(s, sl);
}

// Team wait for row pair u: the records are polled until every member has
// published (or the bounded wait expires, or the test flag
// SV_FLAG_TEAM_WAIT_GIVE_UP asks for no wait at all).  Then the members'
// states are combined into the row log2 normalisers; a member whose wait
// expired takes them from the two full rows instead.  Member 0 also stores
// the row states in its slots.
template <typename E, bool SH>
__device__ __forceinline__ void team_wait_comm(const VerifyParams& p, const UnitDesc& u,
                                               TeamLds& L, int b, int team, int member,
                                               bool& failed) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nt = p.team;
  const uint32_t need = (uint32_t)(u.ordinal + 1);
  const bool give_up = (p.flags & SV_FLAG_TEAM_WAIT_GIVE_UP) != 0u;
  auto complete = [&](const TeamPoll& q) {
    bool mine = true;
#pragma unroll
    for (int k = 0; k < 4; ++k) mine = mine && (uint32_t)(q.w[k] >> 32) == need;
    return __all(lane >= nt || mine) != 0;
  };
  TeamPoll t{};
  bool done = false;
  if (!give_up) {
    t = team_poll(p, u, team);
    done = complete(t);
    const uint32_t limit = failed ? 1u : kSpinLimit;
    for (uint32_t spin = 0; !done && spin < limit; ++spin) {
      __builtin_amdgcn_s_sleep(1);
      t = team_poll(p, u, team);
      done = complete(t);
    }
  }
  const float sl = u.sl;
  SoftmaxPart a{-INFINITY, 0.0f}, c{-INFINITY, 0.0f};
  if (!done) {
    if (!failed && lane == 0)
      __hip_atomic_store(p.sync_error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    failed = true;
    const PlanItem* it = p.plan_pairs + ((int64_t)team + (int64_t)p.nteams * u.ordinal);
    const int64_t trow = it->trow, drow = it->drow;
    a = wave_row_state<E, SH>(p, false, trow, sl);
    c = wave_row_state<E, SH>(p, true, drow, sl);
  } else {
    if (lane < nt) {
      a = SoftmaxPart{__uint_as_float((uint32_t)t.w[0]), __uint_as_float((uint32_t)t.w[1])};
      c = SoftmaxPart{__uint_as_float((uint32_t)t.w[2]), __uint_as_float((uint32_t)t.w[3])};
    }
    float none = 0.0f;
    wave_merge_ref2(a, c, true, none, sl);
  }
  if (lane == 0) {
    // Member 0 stores the row states the team's rates were taken against
    // (the slots keep every member's slice state, which the draw uses).
    if (member == 0) {
      const int64_t unit = (int64_t)(u.code >> 7) * (p.D + 1) + (u.code & 127u);
      p.pair_p[unit] = make_float2(a.m, a.z);
      p.pair_q[unit] = make_float2(c.m, c.z);
    }
    const bool ok = a.m == a.m && c.m == c.m && fabsf(a.m) < INFINITY && fabsf(c.m) < INFINITY;
    L.ok[b] = ok;
    // The references the merges leave (lane maxima, not the row's) can sit
    // far below the row's peak, with sums up to 2^100, whose log2 would
    // carry an ulp of up to 8e-6: the row values are split instead into a
    // reference c near them and a small remainder lz.
    float cp = 0.0f, lzp = 0.0f, cq = 0.0f, lzq = 0.0f;
    if (ok) {
      log2_value(a, sl, cp, lzp);
      log2_value(c, sl, cq, lzq);
    }
    L.c[b][0] = cp;
    L.c[b][1] = cq;
    L.lz[b][0] = lzp;
    L.lz[b][1] = lzq;
    // the second pass's per-thread factors are these times exact powers of 2
    L.ep[b] = exp2_fast(-lzp);
    L.rq[b] = exp2_fast(lzp - lzq);
  }
}

// Sum of the data waves' second-pass sums into the partial slot.
__device__ __forceinline__ void second_pass_comm(const VerifyParams& p, const UnitDesc& u,
                                                 const TeamLds& L, int b, int member) {
  const int lane = threadIdx.x & (kWave - 1);
  float a = (lane < kDataWaves) ? L.acc[b][lane] : 0.0f;
  a = wave_sum(a);
  if (lane == 0) p.part_a[unit_slot(p, u, member)] = a;
}

// ---------------------------------------------------------------------------

template <typename E, int NV, bool SH>
__global__ __launch_bounds__(kTeamThreads) void k_rowteam(VerifyParams p) {
  __shared__ TeamLds L;
  const int nt = p.team;
  const int team = (int)blockIdx.x / nt;
  const int member = (int)blockIdx.x % nt;
  const int64_t n_pairs = p.plan_counts[0];
  const int64_t n_singles = p.plan_counts[1];
  // workgroups past the last whole team have no work
  const bool in_team = team < p.nteams;
  const int64_t my_pairs =
      (in_team && n_pairs > team) ? (n_pairs - 1 - team) / p.nteams + 1 : 0;
  const int64_t my_singles =
      (in_team && n_singles > team) ? (n_singles - 1 - team) / p.nteams + 1 : 0;
  constexpr int PS = SH ? 1 : 2;  // single rows per unit
  const int64_t n = my_pairs + single_units(my_singles, PS);
  const Slice sc = make_slice<E, SH>(p, member);
  // Who publishes a row pair to the team.  The communication wave, after
  // the step's barrier, waits for its own stores before its first poll
  // returns (vector memory operations complete in order); the last data wave
  // to finish the pair publishes before the barrier and leaves the polls
  // free, but its stores queue behind its row loads.  Measured on one
  // MI355X: fp32 rows (V = 262144, rows at 3.9 TB/s) 249 -> 198 us with the
  // data wave publishing and the next unit's loads issued after it; bf16
  // rows (V = 151936, 4.4 TB/s) 147 -> 166 us, so bf16 keeps the
  // communication wave.
  constexpr bool kDataPublish = E::kPerVec == 4;
  if constexpr (kDataPublish) {
    if (threadIdx.x == 0) L.arrived[0] = L.arrived[1] = 0;
    lds_barrier();
  }

  // Both roles run steps s = 0 .. n with one barrier each, then a last one.
  // Data step s: loads of unit s + 2, first pass of unit s, the
  // exponentials of unit s - 1 taken out of the parking slot and those of
  // unit s parked there, barrier, second pass of unit s - 1.  Communication window s
  // (between barriers s and s + 1): sum of the second pass of unit s - 2,
  // combination and publication of the first pass of unit s, team wait for
  // unit s.
  constexpr int kPark = 2 * NV * E::kPerVec / 4;
  __shared__ uint4 park[kPark][kDataThreads];
  if (threadIdx.x < kDataThreads) {
    const uint4* dummy = neg_inf_line<E>();
    LanePtrs<NV> lp{};
    if constexpr (SH) lp = lane_ptrs<E, NV>(p, sc);
    Regs<NV> R0, R1, R2;
    UnitDesc U0 = unit_at(p, 0, n, team, my_pairs, my_singles, PS);
    UnitDesc U1 = unit_at(p, 1, n, team, my_pairs, my_singles, PS);
    UnitDesc U2 = no_unit();
    UnitDesc un = unit_at(p, 2, n, team, my_pairs, my_singles, PS);
    UnitDesc up = no_unit();  // unit s - 1 (parked)
    float mslp1 = 0.0f, mslq1 = 0.0f;
    load_unit<E, NV, SH, PS>(p, U0, sc, lp, R0, dummy);
    load_unit<E, NV, SH, PS>(p, U1, sc, lp, R1, dummy);
    // Step s: first pass on buffer s mod 3, loads into buffer s + 2 mod 3.
    auto step = [&](int64_t s, const Regs<NV>& Rf, const UnitDesc& Uf, Regs<NV>& Rl,
                    UnitDesc& Ul) {
      if constexpr (!kDataPublish) {
        Ul = un;
        load_unit<E, NV, SH, PS>(p, Ul, sc, lp, Rl, dummy);
        un = unit_at(p, s + 3, n, team, my_pairs, my_singles, PS);
      }
      float e[2 * NV * E::kPerVec];
      float mslp = 0.0f, mslq = 0.0f;
      first_pass_data<E, NV, PS>(p, Uf, sc, Rf, L, (int)(s & 1), e, mslp, mslq,
                                 team_single(p, team, PS * (s - my_pairs) + 1));
      // Swap: unit s - 1 out of the parking slot, unit s in (each thread
      // overwrites only the entries it has just read), before the barrier so
      // that the LDS traffic overlaps the other waves' first passes.
      uint4 ex[kPark];
      if (wants_alpha(p, up)) {
#pragma unroll
        for (int k = 0; k < kPark; ++k) ex[k] = park[k][threadIdx.x];
      }
      if (wants_alpha(p, Uf)) {
#pragma unroll
        for (int k = 0; k < kPark; ++k)
          park[k][threadIdx.x] = make_uint4(__float_as_uint(e[4 * k]), __float_as_uint(e[4 * k + 1]),
                                            __float_as_uint(e[4 * k + 2]),
                                            __float_as_uint(e[4 * k + 3]));
        if constexpr (kDataPublish) arrive_pair(p, Uf, L, (int)(s & 1), team, member);
      }
      if constexpr (kDataPublish) {
        // the next unit's loads after the publication, which would otherwise
        // queue behind them
        Ul = un;
        load_unit<E, NV, SH, PS>(p, Ul, sc, lp, Rl, dummy);
        un = unit_at(p, s + 3, n, team, my_pairs, my_singles, PS);
      }
      lds_barrier();
      if (wants_alpha(p, up))
        second_pass_data<E, NV>(p, up, sc, ex, L, (int)((s - 1) & 1), mslp1, mslq1);
      up = Uf;
      mslp1 = mslp;
      mslq1 = mslq;
    };
    for (int64_t s = 0;; s += 3) {
      step(s, R0, U0, R2, U2);
      if (s + 1 > n) break;
      step(s + 1, R1, U1, R0, U0);
      if (s + 2 > n) break;
      step(s + 2, R2, U2, R1, U1);
      if (s + 3 > n) break;
    }
    lds_barrier();
  } else {
    // The communication wave's short dependent chains gate every step; it
    // issues ahead of the data waves that share its SIMD.
    __builtin_amdgcn_s_setprio(3);
    const int lane = threadIdx.x & (kWave - 1);
    // Work items of units base .. base + 63, one per lane (code, T, log2(e)/T;
    // blk2 the second row of a single unit), loaded with vector loads per lane
    // for 64 steps: a scalar load per step would be waited for at every
    // barrier.
    uint4 blk = make_uint4(0u, 0u, 0u, 0u), blk2 = make_uint4(0u, 0u, 0u, 0u);
    auto load_block = [&](int64_t base) {
      const int64_t j = base + lane;
      blk = make_uint4(0u, 0u, 0u, 0u);
      blk2 = make_uint4(0u, 0u, 0u, 0u);
      if (j < n) {
        if (j < my_pairs) {
          const PlanItem* it = p.plan_pairs + ((int64_t)team + (int64_t)p.nteams * j);
          blk = *reinterpret_cast<const uint4*>(&it->code);
        } else {
          const int64_t m = PS * (j - my_pairs);
          blk = *reinterpret_cast<const uint4*>(&p.plan_singles[team_single(p, team, m)].code);
          if (PS == 2 && m + 1 < my_singles)
            blk2 = *reinterpret_cast<const uint4*>(&p.plan_singles[team_single(p, team, m + 1)].code);
        }
      }
      // Wait for the block here, once per 64 steps: the compiler cannot
      // track this conditional load across iterations and would otherwise
      // wait for every outstanding load (the team polls) before each read.
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    };
    auto comm_unit = [&](int64_t s) {
      if (s >= n) return no_unit();
      const int l = (int)(s & 63);
      UnitDesc u;
      u.trow = 0;
      u.drow = 0;
      u.code = (uint32_t)__builtin_amdgcn_readlane((int)blk.x, l);
      const float T = __int_as_float(__builtin_amdgcn_readlane((int)blk.y, l));
      u.sl = __int_as_float(__builtin_amdgcn_readlane((int)blk.z, l));
      u.kind = (s < my_pairs) ? 1 : (T == 0.0f ? 3 : 2);
      u.ordinal = (s < my_pairs) ? (int32_t)s : 0;
      return u;
    };
    auto comm_second = [&](int64_t s) {
      SecondRow r{0u, 0.0f, 0};
      if (PS == 2 && s < n && s >= my_pairs && 2 * (s - my_pairs) + 1 < my_singles) {
        const int l = (int)(s & 63);
        r.code = (uint32_t)__builtin_amdgcn_readlane((int)blk2.x, l);
        const float T2 = __int_as_float(__builtin_amdgcn_readlane((int)blk2.y, l));
        r.sl = __int_as_float(__builtin_amdgcn_readlane((int)blk2.z, l));
        r.kind = (T2 == 0.0f) ? 3 : 2;
      }
      return r;
    };
    bool failed = false;
    UnitDesc um2 = no_unit(), um1 = no_unit();
    for (int64_t s = 0; s <= n; ++s) {
      lds_barrier();
      if ((s & 63) == 0) load_block(s);
      const UnitDesc u = comm_unit(s);
      first_pass_comm<kDataPublish>(p, u, comm_second(s), L, (int)(s & 1), team, member, um2,
                      (int)((s - 2) & 1));
      if (wants_alpha(p, u)) team_wait_comm<E, SH>(p, u, L, (int)(s & 1), team, member, failed);
      um2 = um1;
      um1 = u;
    }
    lds_barrier();
    // um2 is now unit n - 1
    if (wants_alpha(p, um2)) second_pass_comm(p, um2, L, (int)((n - 1) & 1), member);
  }
}

// Team geometry for a row of V elements: NV <= 2 (bf16) or 3 (fp32) 16-byte
// vectors per data thread per row (three buffers of two rows stay in
// registers, the exponentials of one more row pair are parked in LDS), T
// members per row.
// Returns false if a row needs more than 64 members (the caller then uses
// the streaming row pass).  Vocabulary shards do not change it: the members
// tile the concatenated row.
bool team_geometry(sv_dtype dtype, int64_t V, int grid, int32_t* T, int32_t* NV,
                   int32_t* slice_len) {
  const int64_t vec = (dtype == SV_DTYPE_BF16) ? 8 : 4;
  const int64_t rowvec = (V + vec - 1) / vec;
  // fp32 rows take up to three vectors per thread (the registers and the
  // parked exponentials of three 4-element vectors fit), bf16 rows two
  const int64_t nv_max = (dtype == SV_DTYPE_FP32) ? 3 : 2;
  int64_t nv = (rowvec + kDataThreads - 1) / kDataThreads;
  if (nv > nv_max) nv = nv_max;
  if (nv < 1) nv = 1;
  const int64_t t = (rowvec + kDataThreads * nv - 1) / (kDataThreads * nv);
  if (t > 64 || t > grid) return false;
  const int64_t svec = (rowvec + t - 1) / t;
  *T = (int32_t)t;
  *NV = (int32_t)((svec + kDataThreads - 1) / kDataThreads);
  *slice_len = (int32_t)(svec * vec);
  return true;
}

// The team kernel needs every workgroup of a team resident at once.  The grid
// is at most one workgroup per CU and the kernel must fit at least one
// workgroup per CU (checked once per variant), so on a device that is not
// running other work every workgroup is resident from the start.  (A plain
// launch: the cooperative launch path costs more than ten microseconds of
// launch latency here.)  On a shared device the team wait is still bounded.
template <typename E, int NV, bool SH>
static hipError_t launch_team_t(VerifyParams& p, int grid, hipStream_t stream) {
  static std::atomic<int> per_cu{-1};
  int fit = per_cu.load(std::memory_order_relaxed);
  if (fit < 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_rowteam<E, NV, SH>, kTeamThreads, 0) !=
        hipSuccess)
      nb = 0;
    fit = nb;
    per_cu.store(fit, std::memory_order_relaxed);
  }
  if (fit < 1) return hipErrorLaunchOutOfResources;
  hipLaunchKernelGGL((k_rowteam<E, NV, SH>), dim3((unsigned)grid), dim3(kTeamThreads), 0, stream,
                     p);
  return hipGetLastError();
}

template <bool SH>
static hipError_t launch_rowteam_sh(VerifyParams& p, int grid, int nv, hipStream_t stream) {
  if (p.dtype == SV_DTYPE_BF16)
    return nv == 1 ? launch_team_t<Bf16, 1, SH>(p, grid, stream)
                   : launch_team_t<Bf16, 2, SH>(p, grid, stream);
  if (nv == 3) return launch_team_t<F32, 3, SH>(p, grid, stream);
  return nv == 1 ? launch_team_t<F32, 1, SH>(p, grid, stream)
                 : launch_team_t<F32, 2, SH>(p, grid, stream);
}

hipError_t launch_rowteam(VerifyParams& p, int grid, int nv, hipStream_t stream) {
  return p.nshard > 1 ? launch_rowteam_sh<true>(p, grid, nv, stream)
                      : launch_rowteam_sh<false>(p, grid, nv, stream);
}

}  // namespace sv
