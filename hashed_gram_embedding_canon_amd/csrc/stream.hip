// Plain device-to-device copy: the achievable-bandwidth reference that the
// memory-bound kernels of the path are compared with.  One 16-byte piece per
// lane, one pass over the buffer, non-temporal loads and stores: of 1, 2, 4
// and 8 pieces per lane, with and without the non-temporal hint, in one pass
// or grid-stride, this was the fastest (6.48 TB/s read + write over 1 GiB;
// 4 plain pieces per lane: 5.65 TB/s).
#include "kernels.h"

namespace engram {

constexpr int kCopyPer = 1;

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, uint64_t n16) {
  const uint64_t base = (uint64_t)blockIdx.x * (256 * kCopyPer) + threadIdx.x;
  u32x4 v[kCopyPer];
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const uint64_t i = base + (uint64_t)u * 256;
    if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const uint64_t i = base + (uint64_t)u * 256;
    if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
  }
}

hipError_t launch_stream_copy(void* dst, const void* src, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const uint64_t blocks = (n16 + 256 * kCopyPer - 1) / (256 * kCopyPer);
  if (blocks >= (uint64_t(1) << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace engram
