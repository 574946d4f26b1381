// gemm.hpp - dense skinny NVFP4 product y = x W^T (BF16 rows, BF16 out).
//
// One wave per packed tile; the tile stays in registers while the rows pass
// in batches of up to 8.
#pragma once

#include "tile.hpp"

namespace nvfp4moe {

template <int L, int R>
__device__ __forceinline__ void gemm_rows(const TileRegs& T, const uint16_t* __restrict__ x,
                                          int64_t K, int64_t m0, int rows, int col0, int lane,
                                          int64_t tile, int64_t N, float g,
                                          uint16_t* __restrict__ y) {
  uint4 xr[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) load_x_bf16(x, K, m0 + r, r < rows, col0, xr[r]);
  float part[R][8];
  tile_dot_bf16<R>(T, xr, part);
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs<L>(part[r], lane);
  if (!reduced_writer<L>(lane)) return;
  const int64_t rpt = rows_per_tile(L * 32);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= rows) break;
#pragma unroll
    for (int j = 0; j < reduced_count<L>(); ++j) {
      const int64_t n = tile * rpt + tile_row<L>(reduced_slab<L>(lane) + j, lane);
      if (n < N) y[(m0 + r) * N + n] = f32_to_bf16_rne(part[r][j] * g);
    }
  }
}

template <int L>
__global__ void __launch_bounds__(256) skinny_gemm_kernel(const uint16_t* __restrict__ x,
                                                          int64_t M, const uint8_t* __restrict__ w,
                                                          int64_t N, uint16_t* __restrict__ y) {
  constexpr int64_t K = L * 32;
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= tiles_per_matrix(N, K)) return;
  const float g = reinterpret_cast<const float*>(w + gscale_offset(1, N, K))[0];
  TileRegs T;
  load_tile(w + tile * kTileBytes, lane, T);
  const int col0 = 32 * (lane % L);
#pragma unroll 1
  for (int64_t m0 = 0; m0 < M; m0 += 8) {
    opaque_tile(T);
    const int rows = (int)((M - m0) < 8 ? (M - m0) : 8);
    if (rows > 4)
      gemm_rows<L, 8>(T, x, K, m0, rows, col0, lane, tile, N, g, y);
    else if (rows > 2)
      gemm_rows<L, 4>(T, x, K, m0, rows, col0, lane, tile, N, g, y);
    else if (rows > 1)
      gemm_rows<L, 2>(T, x, K, m0, rows, col0, lane, tile, N, g, y);
    else
      gemm_rows<L, 1>(T, x, K, m0, rows, col0, lane, tile, N, g, y);
  }
}

}  // namespace nvfp4moe
