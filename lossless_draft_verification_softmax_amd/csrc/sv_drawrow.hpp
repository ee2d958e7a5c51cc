// sv_drawrow.hpp -- the float32 weights of a draw row, shared by the
// accept-and-draw kernel and the float64 recompute: the residual
// max(0, p - q) after a rejection, or p for the bonus token (the standard
// rejection-sampling rule behind the lossless verification of the
// tradepoint.io page, "Why one universal drafter underperforms").
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_shard.hpp"

namespace sv {

constexpr int kPer = 8;  // consecutive elements per thread and load group
// A float32 draw whose CDF margin (distance of u R to the nearest boundary
// around the drawn token) is below this is recomputed in float64.
constexpr float kDrawMargin32 = 1e-5f;

// Eight consecutive logits starting at i0 (< hi; a multiple of the 16-byte
// vector, 8 bf16 or 4 fp32 elements); entries at or past hi read as -inf,
// which gives them weight 0.  Each 16-byte vector is addressed through the
// row view, so with vocabulary shards (widths a multiple of 8 elements) the
// two fp32 vectors may lie in different shards.
template <typename E, bool SH>
__device__ __forceinline__ void load8(const RowView<E, SH>& row, int64_t i0, int64_t hi,
                                      float (&x)[kPer]) {
  if (i0 + kPer <= hi) {
    if constexpr (E::kPerVec == 8) {
      E::unpack(load16(row.at(i0)), x);
    } else {
      float a[4], b[4];
      E::unpack(load16(row.at(i0)), a);
      E::unpack(load16(row.at(i0 + 4)), b);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = a[j];
        x[4 + j] = b[j];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) x[j] = (i0 + j < hi) ? E::load1(row.at(i0 + j), 0) : -INFINITY;
  }
}

// Eight consecutive logits of the target row and, if has_q, of the draft
// row, in two steps: the raw 16-byte vectors (issued together, so the two
// rows' latencies overlap, and early enough to be in flight while other work
// runs), then the unpacked values a, b as load8 gives them.  A group that
// reaches past hi is read element by element in the second step.
template <typename E>
struct Raw8 {
  static constexpr int NV = kPer / E::kPerVec;  // 16-byte vectors per row
  uint4 x[NV], y[NV];
};

template <typename E, bool SH>
__device__ __forceinline__ void load_raw8(const RowView<E, SH>& prow, const RowView<E, SH>& qrow,
                                          bool has_q, int64_t i0, int64_t hi, Raw8<E>& r) {
  if (i0 + kPer <= hi) {
#pragma unroll
    for (int v = 0; v < Raw8<E>::NV; ++v) r.x[v] = load16(prow.at(i0 + v * E::kPerVec));
    if (has_q) {
#pragma unroll
      for (int v = 0; v < Raw8<E>::NV; ++v) r.y[v] = load16(qrow.at(i0 + v * E::kPerVec));
    }
  }
}

template <typename E, bool SH>
__device__ __forceinline__ void unpack_raw8(const Raw8<E>& r, const RowView<E, SH>& prow,
                                            const RowView<E, SH>& qrow, bool has_q, int64_t i0,
                                            int64_t hi, float (&a)[kPer], float (&b)[kPer]) {
  if (i0 + kPer <= hi) {
#pragma unroll
    for (int v = 0; v < Raw8<E>::NV; ++v) E::unpack(r.x[v], a + v * E::kPerVec);
    if (has_q) {
#pragma unroll
      for (int v = 0; v < Raw8<E>::NV; ++v) E::unpack(r.y[v], b + v * E::kPerVec);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      a[j] = (i0 + j < hi) ? E::load1(prow.at(i0 + j), 0) : -INFINITY;
      if (has_q) b[j] = (i0 + j < hi) ? E::load1(qrow.at(i0 + j), 0) : -INFINITY;
    }
  }
}

template <typename E, bool SH>
__device__ __forceinline__ void load8_pair(const RowView<E, SH>& prow, const RowView<E, SH>& qrow,
                                           bool has_q, int64_t i0, int64_t hi, float (&a)[kPer],
                                           float (&b)[kPer]) {
  Raw8<E> r;
  load_raw8<E, SH>(prow, qrow, has_q, i0, hi, r);
  unpack_raw8<E, SH>(r, prow, qrow, has_q, i0, hi, a, b);
}

// Float32 weights of a draw row, against the row states of the accept
// kernel: 2^((x sl - R(m)) - log2 z), as the accept ratio takes them.
template <typename E, bool SH>
struct Weights32 {
  RowView<E, SH> prow, qrow;
  bool has_q;  // false: bonus draw (w = p)
  float sl, cp, lzp, cq, lzq;  // references R(m) and log2 sums of the rows
  // weights of eight logits a (target) and b (draft; unused for a bonus draw)
  __device__ __forceinline__ void from(const float (&a)[kPer], const float (&b)[kPer],
                                       float (&w)[kPer]) const {
    if (!has_q) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) w[j] = exp2_fast(__builtin_fmaf(a[j], sl, -cp) - lzp);
      return;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float pv = exp2_fast(__builtin_fmaf(a[j], sl, -cp) - lzp);
      const float qv = exp2_fast(__builtin_fmaf(b[j], sl, -cq) - lzq);
      w[j] = fmaxf(pv - qv, 0.0f);
    }
  }
  __device__ __forceinline__ void operator()(int64_t i0, int64_t hi, float (&w)[kPer]) const {
    float a[kPer], b[kPer];
    load8_pair<E, SH>(prow, qrow, has_q, i0, hi, a, b);
    from(a, b, w);
  }
};

// log2(Zq / Zp) from the float32 row states, with Z = sum 2^((x - m) sl): each
// log2 sum lz is taken against the integer reference R(m), so each adds its
// offset R(m) - m sl (exact in float64, as the product of two floats is).
__device__ __forceinline__ double log2_ratio_exact(const DrawState& st) {
  const double op = (double)ref_of(st.mp, st.sl) - (double)st.mp * (double)st.sl;
  const double oq = (double)ref_of(st.mq, st.sl) - (double)st.mq * (double)st.sl;
  return ((double)st.lzq + oq) - ((double)st.lzp + op);
}

template <typename E, bool SH>
__device__ __forceinline__ Weights32<E, SH> weights32(const VerifyParams& p, const DrawState& st) {
  Weights32<E, SH> w;
  w.has_q = st.mode == kDrawResidual;
  w.prow = row_view<E, SH>(p, false, st.prow);
  w.qrow = row_view<E, SH>(p, true, w.has_q ? st.qrow : 0);
  w.sl = st.sl;
  w.cp = ref_of(st.mp, st.sl);
  w.lzp = st.lzp;
  w.cq = ref_of(st.mq, st.sl);
  w.lzq = st.lzq;
  return w;
}

}  // namespace sv
