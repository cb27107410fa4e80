// stream_read: a plain read of one buffer from HBM, the practical ceiling
// the verify kernels' bandwidth is measured against (a kernel that moves
// the same bytes with nothing else to do).
//
// Every work-group reads one contiguous 32 KB block: each of its 256
// threads issues eight independent 16-byte non-temporal loads (addresses
// 4 KB apart, so each load instruction of a wave covers 1 KB contiguously)
// before using any of them, and folds the words with XOR.  A thread stores
// its fold only when it equals a fixed constant, so the loads cannot be
// dropped and the kernel writes (almost) nothing.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "isd_internal.hpp"

namespace isd {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 8;  // 16-byte loads per thread
constexpr size_t kStreamBlock = (size_t)kStreamThreads * kStreamLoads * 16;  // bytes per work-group

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                     size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * (kStreamBlock / 16) + threadIdx.x;
  u32x4 v[kStreamLoads];
#pragma unroll
  for (int u = 0; u < kStreamLoads; ++u) {
    const size_t i = base + (size_t)u * kStreamThreads;
    v[u] = ld16_stream(p + (i < n16 ? i : n16 - 1));
  }
  uint32_t acc = 0u;
#pragma unroll
  for (int u = 0; u < kStreamLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace isd

extern "C" size_t stream_read_sink_words(size_t bytes) {
  return (bytes + isd::kStreamBlock - 1) / isd::kStreamBlock;
}

extern "C" int stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                           void* stream) {
  using namespace isd;
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4))
    return ISD_EINVAL;
  const size_t nwg = (bytes + kStreamBlock - 1) / kStreamBlock;
  if (sink_words < nwg || nwg > 0x7FFFFFFFu) return ISD_EINVAL;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)nwg), dim3(kStreamThreads), 0,
                     (hipStream_t)stream, (const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? ISD_OK : ISD_EHIP;
}
