// sv_device.hpp -- device helpers shared by the specverify kernels (gfx950).
//
// Wave64 cross-lane reductions use DPP row operations for the 16-lane rows
// and the gfx950 permlane swaps across rows; 16-byte vector loads feed the
// streaming loops.  Nothing here allocates or synchronises the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Element access.  bfloat16 is the upper half of an IEEE float32, so a packed
// pair widens with one shift (low half) or one mask (high half).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct Bf16 {
  using Storage = uint16_t;
  static constexpr int kPerVec = 8;  // elements per 16-byte load
  static constexpr uint32_t kNegInfWord = 0xff80ff80u;  // two bf16 -inf
  __device__ static __forceinline__ float load1(const Storage* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
  __device__ static __forceinline__ void unpack(const uint4& v, float f[8]) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
  }
};

struct F32 {
  using Storage = float;
  static constexpr int kPerVec = 4;
  static constexpr uint32_t kNegInfWord = 0xff800000u;  // fp32 -inf
  __device__ static __forceinline__ float load1(const Storage* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void unpack(const uint4& v, float f[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

// One 16-byte vector of a logit row.  Rows are read once, so the loads are
// non-temporal: they do not allocate the lines in the Infinity Cache or L2,
// whose fills would otherwise compete with the stream (a plain streaming read
// of 642 MB on one MI355X: 7.1 TB/s this way, 6.2 TB/s with ordinary loads).
__device__ __forceinline__ uint4 load16(const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 v;
  v.x = __builtin_nontemporal_load(&q->x);
  v.y = __builtin_nontemporal_load(&q->y);
  v.z = __builtin_nontemporal_load(&q->z);
  v.w = __builtin_nontemporal_load(&q->w);
  return v;
}

// The same with an ordinary load, for rows that are read again soon (the
// streaming row pass's second pass over a pair).
__device__ __forceinline__ uint4 load16_keep(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// IEEE 754-2019 maximum (NaN-propagating): v_maximum3_f32 on gfx950, so a
// NaN anywhere in a row survives into its maximum.
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Raw hardware 2^x (v_exp_f32): about 1 ulp; results below 2^-126 may flush,
// which is far under what any sum here can resolve.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Cross-lane exchange.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16 lanes

// The other row of a row pair (lanes 0-15 <-> 16-31, 32-47 <-> 48-63) and
// the other half of the wave (0-31 <-> 32-63), via the gfx950 permlane
// swaps.  Each swap returns the two operands with rows exchanged; combining
// both results gives every lane the pair's two values.
template <typename Op>
__device__ __forceinline__ float combine_rows16(float v, Op op) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float combine_halves32(float v, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// All-reduce of a commutative, associative op across the 64 lanes; every lane
// gets the result.  The reduction tree is fixed, so results are reproducible.
template <typename Op>
__device__ __forceinline__ float wave_allreduce(float v, Op op) {
  v = op(v, dpp_f<kDppQuadXor1>(v));
  v = op(v, dpp_f<kDppQuadXor2>(v));
  v = op(v, dpp_f<kDppHalfMirror>(v));
  v = op(v, dpp_f<kDppMirror>(v));
  v = combine_rows16(v, op);
  v = combine_halves32(v, op);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_allreduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_allreduce(v, [](float a, float b) { return vmax(a, b); });
}

// Shuffle-based fallback for 64-bit payloads (ds_bpermute, no LDS storage).
__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
  int2 p = *reinterpret_cast<int2*>(&v);
  p.x = __shfl_xor(p.x, mask);
  p.y = __shfl_xor(p.y, mask);
  return *reinterpret_cast<double*>(&p);
}

// ---------------------------------------------------------------------------
// Online softmax state over a row slice, in the log2 domain: the slice's
// maximum m (raw logit units) and z = sum 2^(x sl - R(m)), sl = log2(e) / T,
// with the integer reference R(m) = rint(fl(m sl)).  Every exponential of a
// row is taken against such a reference (one fused x sl - R, rounded once;
// its argument is at most 1/2 at the maximum), and every rescale and every
// normaliser uses the same references, so the value of a state is exactly
// z 2^R(m) at any magnitude of m sl.  Two references differ by an exact
// integer: a merge rescales by 2^(R(a) - R(m)) without rounding, whichever of
// a and m is larger (with references fl(m sl) the difference rounds once the
// two are more than a factor 2 apart, as when a lane holding a T = 1 row's
// peak is merged against another lane's maximum, and mixing in the exact
// product m sl biases every p by 2^(m sl - fl(m sl)), up to 1e-5 relative
// once |m sl| passes 128).
struct SoftmaxPart {
  float m;
  float z;
};

// The integer reference R(m) = rint(fl(m sl)) of a state with maximum m
// (exact as a float while |m sl| < 2^24; -inf and NaN pass through).
__device__ __forceinline__ float ref_of(float m, float sl) {
#pragma clang fp contract(off)
  return __builtin_rintf(m * sl);
}

// The references carry a row state exactly while |fl(m sl)| < 2^24: then
// R(m) lies within 3/4 of m sl, so x sl - R(m) is within [-3/4, 3/4] at the
// maximum (past 2^24 the rounding of fl(m sl) alone can exceed the range of
// 2^x).  A row whose scaled maximum reaches 2^24 (a
// temperature below about 1e-5 for logits of magnitude 100) is outside the
// verifier's domain: its request is reported invalid (SV_BIT_BAD_TEMPERATURE).
constexpr float kMaxScaledMax = 16777216.0f;  // 2^24
__device__ __forceinline__ bool scale_ok(float m, float sl) {
  return fabsf(m * sl) < kMaxScaledMax;
}

// 2^(R(a) - R(m)): the factor that takes a sum relative to a's reference to
// m's reference (exactly 1 for a = m; the exponent is an exact integer).
__device__ __forceinline__ float rescale(float a, float m, float sl) {
  return exp2_fast(ref_of(a, sl) - ref_of(m, sl));
}

// Merge of two partial states (the associative (max, rescaled sum) rule).
__device__ __forceinline__ SoftmaxPart merge_parts(SoftmaxPart a, SoftmaxPart b, float sl) {
  float m = vmax(a.m, b.m);
  if (m == -INFINITY) return {m, 0.0f};
  // A part whose max is -inf holds only masked entries: it adds nothing.
  float za = (a.m == -INFINITY) ? 0.0f : a.z * rescale(a.m, m, sl);
  float zb = (b.m == -INFINITY) ? 0.0f : b.z * rescale(b.m, m, sl);
  return {m, za + zb};
}

__device__ __forceinline__ SoftmaxPart wave_merge(SoftmaxPart p, float sl) {
  float m = wave_max(p.m);
  float z = (p.m == -INFINITY || m == -INFINITY) ? 0.0f : p.z * rescale(p.m, m, sl);
  // NaN maxima propagate through vmax; keep the NaN so the row reads invalid.
  if (m != m) z = m;
  return {m, wave_sum(z)};
}

// The same merge with the maximum taken by v_max_f32, which the compiler
// fuses with the DPP lane moves (the NaN-propagating maximum cannot be);
// a NaN maximum in any lane is carried by a ballot instead.
__device__ __forceinline__ SoftmaxPart wave_merge_fast(SoftmaxPart p, float sl) {
  const bool nan = __ballot(p.m != p.m) != 0ull;
  float m = wave_allreduce(p.m, [](float a, float b) { return fmaxf(a, b); });
  float z = (p.m == -INFINITY || m == -INFINITY) ? 0.0f : p.z * rescale(p.m, m, sl);
  z = wave_sum(z);
  if (nan) {
    m = __int_as_float(0x7fc00000);
    z = m;
  }
  return {m, z};
}

// Wave merge against lane 0's maximum instead of the wave maximum: each sum
// is rescaled to 2^R(m_0), which needs no max reduction.  The result
// (m_0, z) is a valid state whether or not m_0 is the largest element: its
// value is z 2^R(m_0).  A rescaled sum above 2^100 (or NaN), a non-finite
// m_0 or an empty lane 0 takes the exact merge instead.  So every element x
// under a merged state satisfies (x - m) sl <= 106, through any number of
// such merges, and sums stay far from float32 overflow.
__device__ __forceinline__ SoftmaxPart wave_merge_ref(SoftmaxPart p, float sl) {
  const float m0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.m)));
  const bool empty = p.m == -INFINITY;
  const float zs = empty ? 0.0f : p.z * rescale(p.m, m0, sl);
  if (__ballot(!(zs <= 0x1p100f)) != 0ull || !(fabsf(m0) < INFINITY))
    return wave_merge_fast(p, sl);
  return {m0, wave_sum(zs)};
}

// The same state against a reference near its log2 normaliser: (m', z') with
// z' 2^R(m') = z 2^R(m) and z' in about [0.5, 1), so that log2 z' is small
// and exact to about 1e-7, whatever reference the merges used (merges
// against lane 0's maximum leave sums up to 2^100, and one float32 ulp of a
// log2 near 100 is 8e-6: up to 1e-5 relative in every p taken from it).
// With z = mant 2^k (exact), c = fl(R(m) + k) and its rounding error e
// (two-sum; 0 while |R(m)| < 2^23): z 2^R(m) = mant 2^(c + e); m' = c / sl
// (to within an ulp or two: any m' with R(m') near c will do) and
// z' = mant 2^((c - R(m')) + e).  Empty, zero-sum or non-finite states, and
// products out of range, are returned unchanged.
__device__ __forceinline__ SoftmaxPart renormalise(SoftmaxPart s, float sl) {
#pragma clang fp contract(off)
  const float r0 = ref_of(s.m, sl);
  if (!(s.z > 0.0f) || !(s.z < INFINITY) || !(fabsf(r0) < 0x1p100f)) return s;
  int k;
  const float mant = frexpf(s.z, &k);
  const float kf = (float)k;
  const float c = r0 + kf;
  const float bb = c - r0;
  const float e = (r0 - (c - bb)) + (kf - bb);
  const float m1 = c * __builtin_amdgcn_rcpf(sl);
  if (!(fabsf(m1) < INFINITY)) return s;
  const float c1 = ref_of(m1, sl);
  return {m1, mant * exp2_fast((c - c1) + e)};
}

// A state's log2 value R(m) + log2 z as a reference c near it plus a small
// remainder lz, exact to about 1e-7 whatever reference the merges used: with
// z = mant 2^k (exact), c = fl(R(m) + k), e its rounding error (two-sum; 0
// while |R(m)| < 2^23) and lz = log2(mant) + e.  For a state with z > 0 and
// a finite product m sl.
__device__ __forceinline__ void log2_value(SoftmaxPart s, float sl, float& c, float& lz) {
#pragma clang fp contract(off)
  int k;
  const float mant = frexpf(s.z, &k);
  const float r0 = ref_of(s.m, sl);
  const float kf = (float)k;
  c = r0 + kf;
  const float bb = c - r0;
  lz = __log2f(mant) + ((r0 - (c - bb)) + (kf - bb));
}

// Three wave sums over the same fixed tree, interleaved so that their
// dependent chains overlap.
__device__ __forceinline__ void wave_sum3(float& a, float& b, float& c) {
  auto step = [&](auto f) {
    a = a + f(a);
    b = b + f(b);
    c = c + f(c);
  };
  step([](float v) { return dpp_f<kDppQuadXor1>(v); });
  step([](float v) { return dpp_f<kDppQuadXor2>(v); });
  step([](float v) { return dpp_f<kDppHalfMirror>(v); });
  step([](float v) { return dpp_f<kDppMirror>(v); });
  auto plus = [](float x, float y) { return x + y; };
  a = combine_rows16(a, plus);
  b = combine_rows16(b, plus);
  c = combine_rows16(c, plus);
  a = combine_halves32(a, plus);
  b = combine_halves32(b, plus);
  c = combine_halves32(c, plus);
}

// wave_merge_ref on two states (q may be absent) and a plain wave sum, with
// one fallback branch for both states: three independent reduction chains.
__device__ __forceinline__ void wave_merge_ref2(SoftmaxPart& p, SoftmaxPart& q, bool has_q,
                                                float& sum, float sl) {
  const float m0p = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.m)));
  const float m0q = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(q.m)));
  float zp = (p.m == -INFINITY) ? 0.0f : p.z * rescale(p.m, m0p, sl);
  float zq = (!has_q || q.m == -INFINITY) ? 0.0f : q.z * rescale(q.m, m0q, sl);
  const bool bad_lane = !(zp <= 0x1p100f) || !(zq <= 0x1p100f);
  if (__ballot(bad_lane) != 0ull || !(fabsf(m0p) < INFINITY) ||
      (has_q && !(fabsf(m0q) < INFINITY))) {
    p = wave_merge_fast(p, sl);
    if (has_q) q = wave_merge_fast(q, sl);
    sum = wave_sum(sum);
    return;
  }
  wave_sum3(zp, zq, sum);
  p = {m0p, zp};
  if (has_q) q = {m0q, zq};
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies whose high words are xored with the other two counter
// words and the round key, the key advancing by the Weyl increments
// 0x9E3779B9 (golden ratio) and 0xBB67AE85 (sqrt 3 - 1) between rounds.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint32_t a_lo = 0xD2511F53u * c0;
    const uint32_t a_hi = __umulhi(0xD2511F53u, c0);
    const uint32_t b_lo = 0xCD9E8D57u * c2;
    const uint32_t b_hi = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = b_hi ^ c1 ^ k0;
    const uint32_t n2 = a_hi ^ c3 ^ k1;
    c0 = n0;
    c1 = b_lo;
    c2 = n2;
    c3 = a_lo;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {{c0, c1, c2, c3}};
}

// Uniform on the 2^-24 grid from the top 24 bits of a word (exact in fp32).
__device__ __forceinline__ float u24(uint32_t w) {
  return static_cast<float>(w >> 8) * (1.0f / 16777216.0f);
}

}  // namespace sv
