// stream_copy.hip -- measurement probes.  A plain streaming copy with the row
// kernels' memory access pattern (16-byte buffer loads and stores with the same cache
// policy, a one-shot grid of 256-lane workgroups).  It computes nothing: its
// bandwidth is the practical HBM ceiling that the norm and RoPE kernels,
// which read and write each byte once, are measured against.  Of 1, 2, 4
// and 8 vectors per lane, one (the most workgroups, each lane's load and
// store back to back) copied fastest on MI355X: about 6.65 TB/s over
// 2 x 671 MB with the streaming store policy.
#include "nr_device.hpp"
#include "nr_internal.hpp"

namespace nr {

// One 16-byte vector per lane; each workgroup's buffer range covers its own
// 4 KiB, so the last one's tail (and copies past 4 GiB) need no index math.
__global__ void __launch_bounds__(256) stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t first = static_cast<int64_t>(blockIdx.x) * 256;
  const uint32_t bytes = static_cast<uint32_t>(min(nvec - first, int64_t{256}) * 16);
  const rsrc_t sr = make_rsrc(src + first, bytes);
  const rsrc_t dr = make_rsrc(dst + first, bytes);
  const uint32_t off = threadIdx.x * 16u;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, kStream),
                                         dr, off, 0, kStreamStore);
}

// Two streams read, one written (dst = a ^ b, the backward's 2:1 mix), or
// two streams read and nothing written (a word per workgroup goes to dst only
// if the data were to xor to a fixed pattern, which does not happen for the
// probe's inputs): the practical ceilings of the other read/write mixes the
// kernels use.  One 16-byte vector of each input per lane, as the copy.
template <bool WRITE>
__global__ void __launch_bounds__(256) stream_mix_kernel(const u32x4* __restrict__ a,
                                                         const u32x4* __restrict__ b,
                                                         u32x4* __restrict__ dst, int64_t nvec) {
  const int64_t first = static_cast<int64_t>(blockIdx.x) * 256;
  const uint32_t bytes = static_cast<uint32_t>(min(nvec - first, int64_t{256}) * 16);
  const rsrc_t ar = make_rsrc(a + first, bytes);
  const rsrc_t br = make_rsrc(b + first, bytes);
  const uint32_t off = threadIdx.x * 16u;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, kStream) ^
                  __builtin_amdgcn_raw_buffer_load_b128(br, off, 0, kStream);
  if constexpr (WRITE) {
    __builtin_amdgcn_raw_buffer_store_b128(v, make_rsrc(dst + first, bytes), off, 0, kStreamStore);
  } else {
    if ((v[0] & v[1] & v[2] & v[3]) == 0xffffffffu)  // data-dependent, never for the probe's data
      __builtin_amdgcn_raw_buffer_store_b128(v, make_rsrc(dst + first, bytes), off, 0, 0);
  }
}

hipError_t launch_stream_mix(const void* a, const void* b, void* dst, int64_t nvec, bool write,
                             hipStream_t st) {
  const int64_t blocks = (nvec + 255) / 256;
  auto kern = write ? stream_mix_kernel<true> : stream_mix_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const u32x4*>(a), static_cast<const u32x4*>(b),
                     static_cast<u32x4*>(dst), nvec);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t st) {
  const int64_t blocks = (nvec + 255) / 256;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  return hipGetLastError();
}

}  // namespace nr
