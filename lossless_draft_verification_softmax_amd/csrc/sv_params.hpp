// sv_params.hpp -- kernel entry helper for kernels launched with VerifyParams.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_internal.hpp"

namespace sv {

// Touch every 64-byte line of the kernel's parameter block at entry, so that
// the scalar loads of later phases hit the scalar cache instead of each
// waiting on a miss of its own.  The loads go out together and are waited on
// once, here.
__device__ __forceinline__ void warm_params(const VerifyParams& p) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&p);
  uint32_t acc = 0u;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(VerifyParams) / 4); i += 16) acc ^= w[i];
  asm volatile("" ::"s"(acc));
}

}  // namespace sv
