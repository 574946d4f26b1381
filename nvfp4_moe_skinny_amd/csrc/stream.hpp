// stream.hpp - the read ceiling: one pass over a buffer with the same 16-byte
// nontemporal loads the weight streams use, nothing else. Its rate is the
// bandwidth the products are compared with besides the 8 TB/s peak.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

constexpr int kStreamThreads = 256;
constexpr int64_t kStreamMaxBlocks = 8192;
// 16-byte loads in flight per thread: measured on one pass over cold buffers,
// 1 or 2 per thread (more, smaller workgroups) read 54 MB in 10.3 us where 8
// take 11.9 and 16 take 15.4, and 148 MB in 24.2 us (1) against 26.4 (8);
// at 4 GiB, 8 per thread with at most 8192 workgroups reach 6.7 TB/s (2: 6.3).
constexpr int64_t kStreamLargeBytes = (int64_t)512 << 20;
__host__ __device__ constexpr int stream_unroll(int64_t bytes) {
  return bytes < kStreamLargeBytes ? 1 : 8;
}

// Grid-stride over n 16-byte vectors; block b writes the XOR of the 32-bit
// words it read to sink[b] (so the XOR over sink is the XOR of the buffer).
template <int UNROLL>
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const uint4* __restrict__ src,
                                                                     int64_t n,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = load_stream(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = load_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kStreamThreads / 64];
  // XOR over the block: within each wave by shuffles, then the four waves' values in LDS
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace nvfp4moe
