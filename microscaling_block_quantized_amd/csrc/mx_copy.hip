// A plain device copy, 16 bytes per thread with non-temporal loads and stores:
// the bandwidth ceiling that the casts are compared against (the same read and
// write traffic with no arithmetic). One chunk per thread measured fastest on
// MI355X (6.44 TB/s on 276 MB per launch; 4 or 8 chunks per thread 5.9 / 4.0).
#include "mx_kernels.h"

namespace mx {

namespace {

typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void copy_nt_kernel(const u32x4c* __restrict__ src, u32x4c* __restrict__ dst,
                                                               int64_t chunks) {
  const int64_t i = int64_t(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (i < chunks) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_copy_nt(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t chunks = bytes / 16;
  return launch_kernel(copy_nt_kernel, dim3(uint32_t(copy_blocks(bytes))), dim3(kCopyThreads), s,
                       static_cast<const u32x4c*>(src), static_cast<u32x4c*>(dst), chunks);
}

}  // namespace mx
