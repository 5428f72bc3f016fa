// Streaming-read kernel: the HBM read rate this device reaches with the
// decode kernel's load width (16 bytes per lane) and full occupancy. The
// decode call's roofline is reported against it beside the nominal peak.

#include "stream_read.h"

namespace pkv {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;  // loads in flight per lane

// Workgroup b reads chunks of kStreamThreads * kStreamUnroll 16-byte words in
// a grid-stride loop (each instruction: 4 KiB contiguous per workgroup) and
// folds them into one word per workgroup, written to sink[b] so the loads
// stay live.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                    size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t step = (size_t)kStreamThreads * kStreamUnroll;
  for (size_t base = (size_t)blockIdx.x * step; base < n16; base += (size_t)gridDim.x * step) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * kStreamThreads + threadIdx.x;
      v[u] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  __shared__ uint32_t s_acc[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) a ^= s_acc[w];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream) {
  stream_read_kernel<<<dim3((unsigned)grid), dim3(kStreamThreads), 0, stream>>>(
      static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
