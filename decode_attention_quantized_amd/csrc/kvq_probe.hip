// Streaming-read reference for measurements: how fast a plain read of a
// given number of bytes runs on a given grid of 1024-thread workgroups, so a
// decode call can be compared with the fastest read of the same bytes at the
// same size and launch shape (a small read is bound by latency and launch
// ramp, not by the HBM peak). Not part of the attention path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq.h"

namespace {

constexpr int kProbeThreads = 1024;

// Workgroup g reads the 16-byte pieces [n16 * g / G, n16 * (g + 1) / G),
// consecutive threads on consecutive pieces, four loads in flight per thread,
// and XORs every 32-bit word it read into sink[g].
__global__ __launch_bounds__(kProbeThreads) void stream_read(const uint4* __restrict__ src, int64_t n16,
                                                             uint32_t* sink) {
  const int64_t g = blockIdx.x, G = gridDim.x;
  const int64_t lo = n16 * g / G, hi = n16 * (g + 1) / G;
  constexpr int T = kProbeThreads;
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 3 * T < hi; i += 4 * T) {
    const uint4 v0 = src[i], v1 = src[i + T], v2 = src[i + 2 * T], v3 = src[i + 3 * T];
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < hi; i += T) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), o));
  if ((threadIdx.x & 63) == 0) atomicXor(sink + g, acc);
}

}  // namespace

extern "C" int32_t kvq_stream_read(const void* src, int64_t bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) != 0 || grid <= 0 || grid > (1 << 20)) return KVQ_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0) return KVQ_ERR_ALIGN;
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}
