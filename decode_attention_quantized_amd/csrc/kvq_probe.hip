// Streaming-read reference for measurements: how fast a plain read of a
// given number of bytes runs on a given grid and workgroup size, so a decode
// call can be compared with the fastest read of the same bytes at the same
// size (a small read is bound by latency and launch ramp, not by the HBM
// peak). Not part of the attention path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq.h"

namespace {

constexpr int kInFlight = 8;   // 16-byte loads a thread issues before it uses any of them

// Workgroup g reads the 16-byte pieces [n16 * g / G, n16 * (g + 1) / G),
// consecutive threads on consecutive pieces. A thread issues up to kInFlight
// loads (all of its pieces when the slice is at most kInFlight * T pieces)
// before it consumes the first; the XOR of every 32-bit word the workgroup
// read goes into sink[g].
template <int T>
__global__ __launch_bounds__(T) void stream_read(const uint4* __restrict__ src, int64_t n16, uint32_t* sink) {
  const int64_t g = blockIdx.x, G = gridDim.x;
  const int64_t lo = n16 * g / G, hi = n16 * (g + 1) / G;
  uint32_t acc = 0;
  for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += int64_t(kInFlight) * T) {
    uint4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int64_t i = i0 + int64_t(k) * T;
      v[k] = i < hi ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), o));
  // one atomic per workgroup (atomics of many waves on one address would
  // queue behind each other and time the atomics rather than the read)
  __shared__ uint32_t part[T / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < T / 64; ++w) x ^= part[w];
    atomicXor(sink + g, x);
  }
}

}  // namespace

extern "C" int32_t kvq_stream_read(const void* src, int64_t bytes, int32_t grid, int32_t threads, uint32_t* sink,
                                   void* stream) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) != 0 || grid <= 0 || grid > (1 << 20)) return KVQ_ERR_ARG;
  if (threads != 256 && threads != 512 && threads != 1024) return KVQ_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0) return KVQ_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint4* s = static_cast<const uint4*>(src);
  if (threads == 256) hipLaunchKernelGGL(stream_read<256>, dim3(grid), dim3(256), 0, st, s, bytes / 16, sink);
  else if (threads == 512) hipLaunchKernelGGL(stream_read<512>, dim3(grid), dim3(512), 0, st, s, bytes / 16, sink);
  else hipLaunchKernelGGL(stream_read<1024>, dim3(grid), dim3(1024), 0, st, s, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}
