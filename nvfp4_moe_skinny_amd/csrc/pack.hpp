// pack.hpp - canonical NVFP4 <-> library tile layout, and the decode test hook.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

// One thread per 16-byte chunk of the packed tensor: copies the chunk's codes
// and its two scale bytes from the canonical arrays (zeros for padded rows).
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   const float* __restrict__ g, int64_t G,
                                                   int64_t N, int64_t K, uint8_t* __restrict__ out) {
  const int64_t L = panel_k(K) / 32;
  const int64_t Q = panels(K);
  const int64_t rpt = rows_per_tile(K);
  const int64_t tiles = tiles_per_matrix(N, K);
  const int64_t total = G * tiles * 512;
  const int64_t mbytes = tiles * kTileBytes;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t gi = c / (tiles * 512);
    const int64_t rem = c - gi * tiles * 512;
    const int64_t t = rem / 512;   // row block t / Q, panel t % Q
    const int64_t ct = rem % 512;  // chunk within tile = 64 * slab + lane
    const int64_t slab = ct / 64, lane = ct % 64;
    const int64_t n = (t / Q) * rpt + ct / L;
    const int64_t q = (t % Q) * L + ct % L;  // chunk of the row
    uint8_t* dst = out + gi * mbytes + t * kTileBytes;
    uint8_t* sdst = dst + kTileCodeBytes + lane * 16 + slab * 2;
    if (n < N) {
      const uint8_t* src = codes + (gi * N + n) * (K / 2) + q * 16;
#pragma unroll
      for (int b = 0; b < 16; ++b) dst[ct * 16 + b] = src[b];
      const uint8_t* ssrc = scales + (gi * N + n) * (K / 16) + q * 2;
      sdst[0] = ssrc[0];
      sdst[1] = ssrc[1];
    } else {
#pragma unroll
      for (int b = 0; b < 16; ++b) dst[ct * 16 + b] = 0;
      sdst[0] = 0;
      sdst[1] = 0;
    }
  }
  // tensor scales after the matrices
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < G;
       i += (int64_t)gridDim.x * blockDim.x)
    reinterpret_cast<float*>(out + gscale_offset(G, N, K))[i] = g[i];
}

// One thread per chunk: the 32 elements of a chunk decoded by the same
// routines the products use, written to canonical [G][N][K] positions.
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ packed, int64_t G,
                                                      int64_t N, int64_t K, int apply_g, int path,
                                                      float* __restrict__ out) {
  const int64_t L = panel_k(K) / 32;
  const int64_t Q = panels(K);
  const int64_t rpt = rows_per_tile(K);
  const int64_t tiles = tiles_per_matrix(N, K);
  const int64_t total = G * tiles * 512;
  const int64_t mbytes = tiles * kTileBytes;
  const float* gs = reinterpret_cast<const float*>(packed + gscale_offset(G, N, K));
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t gi = c / (tiles * 512);
    const int64_t rem = c - gi * tiles * 512;
    const int64_t t = rem / 512;
    const int ct = (int)(rem % 512);
    const int slab = ct / 64, lane = ct % 64;
    const int64_t n = (t / Q) * rpt + ct / L;
    if (n >= N) continue;
    const int64_t q = (t % Q) * L + ct % L;  // chunk of the row
    const uint8_t* tile = packed + gi * mbytes + t * kTileBytes;
    const uint4 cv = *reinterpret_cast<const uint4*>(tile + ct * 16);
    const uint4 sv = *reinterpret_cast<const uint4*>(tile + kTileCodeBytes + lane * 16);
    const float s0 = tile_scale(sv, slab, 0), s1 = tile_scale(sv, slab, 1);
    const float gv = gs[gi];
    float* dst = out + (gi * N + n) * K + q * 32;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const uint32_t word = u4_get(cv, p >> 2);
      float a, b;
      if (path == 0) {
        const bf16x2 v = fp4_pair_bf16(word, p & 3);
        a = (float)v[0];
        b = (float)v[1];
      } else {
        const f32x2 v = fp4_pair_f32(word, p & 3);
        a = v[0];
        b = v[1];
      }
      const float s = p < 8 ? s0 : s1;
      a *= s;
      b *= s;
      if (apply_g) {
        a *= gv;
        b *= gv;
      }
      dst[2 * p] = a;
      dst[2 * p + 1] = b;
    }
  }
}

}  // namespace nvfp4moe
