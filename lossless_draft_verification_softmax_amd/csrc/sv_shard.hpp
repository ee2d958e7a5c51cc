// sv_shard.hpp -- element addressing of a logits row that may be split over
// vocabulary shards (sv_verify_batch_sharded): shard s holds columns
// [s W, min(V, (s + 1) W)) of every row in its own buffer, all at the same row
// stride.  W is a multiple of 8 elements, so no 16-byte vector and no group
// of 8 consecutive elements starting at a multiple of 8 crosses a shard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_block.hpp"
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

// A row of the target (draft = false) or draft logits: element i lives at
// at(i).  SH = false: one buffer, the contiguous row (the unsharded kernels
// are instantiated with it and pay nothing for shards).
template <typename E, bool SH>
struct RowView {
  using S = typename E::Storage;
  const S* base;               // the row's first element (one shard)
  const void* const* tab;      // shard pointers (several shards)
  int64_t row, stride, W;
  int32_t nshard;
  __device__ __forceinline__ const S* at(int64_t i) const {
    if constexpr (!SH) return base + i;
    const int64_t s = i / W;
    return static_cast<const S*>(tab[s]) + row * stride + (i - s * W);
  }
};

template <typename E, bool SH>
__device__ __forceinline__ RowView<E, SH> row_view(const VerifyParams& p, bool draft, int64_t row) {
  RowView<E, SH> v;
  v.nshard = p.nshard;
  v.row = row;
  v.stride = p.stride;
  v.W = p.shard_w;
  v.tab = SH ? p.shard_tab + (draft ? kMaxShards : 0) : nullptr;
  v.base = SH ? nullptr : row_ptr<E>(draft ? p.draft : p.target, row, p.stride);
  return v;
}

}  // namespace sv
