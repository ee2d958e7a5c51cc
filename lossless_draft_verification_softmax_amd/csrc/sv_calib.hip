// sv_calib.hip -- a plain streaming read, for calibrating the HBM roofline
// the verification kernels are measured against: the rate at which this chip
// reads a buffer once, with no arithmetic to hide and nothing written back.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// Each thread reads kUnroll 16-byte vectors per iteration (all issued before
// any is used), grid-stride over the buffer, and folds them by xor; one
// 32-bit atomic per workgroup keeps the loads live.  The loads are
// non-temporal, as the verification kernels' row loads are: a buffer read
// once need not be kept in the Infinity Cache or L2 (on one MI355X, 7.1 TB/s
// at one workgroup per CU against 6.2 TB/s with ordinary loads).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  uint4 v;
  v.x = __builtin_nontemporal_load(&p->x);
  v.y = __builtin_nontemporal_load(&p->y);
  v.z = __builtin_nontemporal_load(&p->z);
  v.w = __builtin_nontemporal_load(&p->w);
  return v;
}
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void k_stream_read(const uint4* __restrict__ buf,
                                                              int64_t nvec, uint32_t* sink) {
  __shared__ uint32_t s_acc[kReadThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  uint32_t acc = 0u;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  for (; i + (kReadUnroll - 1) * stride < nvec; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = load_nt(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < nvec; i += stride) {
    const uint4 v = load_nt(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int w = 0; w < kReadThreads / 64; ++w) t ^= s_acc[w];
    atomicXor(sink, t);
  }
}

}  // namespace sv

extern "C" sv_status sv_stream_read(const void* buf, size_t bytes, int32_t blocks_per_cu,
                                    uint32_t* sink, void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes % 16 != 0 ||
      blocks_per_cu < 1 || blocks_per_cu > 32)
    return SV_ERR_INVALID_ARGUMENT;
  if (bytes == 0) return SV_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return SV_ERR_DEVICE;
  const int64_t nvec = (int64_t)(bytes / 16);
  int64_t grid = (int64_t)cus * blocks_per_cu;
  const int64_t need = (nvec + sv::kReadThreads - 1) / sv::kReadThreads;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(sv::k_stream_read, dim3((unsigned)grid), dim3(sv::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), nvec, sink);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_DEVICE;
}
