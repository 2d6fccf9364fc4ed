// stream_copy.hip -- a plain streaming copy with the row kernels' memory
// access pattern (16-byte non-temporal loads and stores, a one-shot grid of
// 256-lane workgroups).  It computes nothing: its bandwidth is the practical
// HBM ceiling that the norm and RoPE kernels, which read and write each byte
// once, are measured against.  Of 1, 2, 4 and 8 vectors per lane, one (the
// most workgroups, each lane's load and store back to back) copied fastest
// on MI355X: about 6.5 TB/s over 2 x 671 MB.
#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

constexpr int kCopyU = 1;  // 16-byte vectors per lane (1, 2, 4, 8 measured: 1 is fastest)

__global__ void __launch_bounds__(256) stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (256 * kCopyU) + threadIdx.x;
  u32x4 v[kCopyU];
#pragma unroll
  for (int u = 0; u < kCopyU; ++u) {
    const int64_t i = base + u * 256;
    if (i < nvec) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyU; ++u) {
    const int64_t i = base + u * 256;
    if (i < nvec) __builtin_nontemporal_store(v[u], dst + i);
  }
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t st) {
  const int64_t per_block = 256 * kCopyU;
  const int64_t blocks = (nvec + per_block - 1) / per_block;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  return hipGetLastError();
}

}  // namespace nr
