// gemm.hpp - dense skinny NVFP4 product y = x W^T (BF16 rows, BF16 out).
//
// One wave per row block of W. With one panel (K a power of two <= 2048) the
// tile stays in registers while the rows pass in batches of up to 8; with Q
// panels the wave streams the row block's Q tiles per batch of rows, adding
// each panel's per-slab partial sums before one reduction.
#pragma once

#include "dense.hpp"

namespace nvfp4moe {

// Reduces R rows' per-slab partial sums and writes rows m0 .. m0 + rows - 1
// of y for row block blk.
template <int L, int R>
__device__ __forceinline__ void gemm_write(float (&part)[R][8], int64_t m0, int rows, int lane,
                                           int64_t blk, int64_t N, float g,
                                           uint16_t* __restrict__ y) {
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs<L>(part[r], lane);
  if (!reduced_writer<L>(lane)) return;
  const int64_t rpt = 16384 / (L * 32);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= rows) break;
#pragma unroll
    for (int j = 0; j < reduced_count<L>(); ++j) {
      const int64_t n = blk * rpt + tile_row<L>(reduced_slab<L>(lane) + j, lane);
      if (n < N) y[(m0 + r) * N + n] = f32_to_bf16_rne(part[r][j] * g);
    }
  }
}

// One panel (the tile held in T): rows m0 .. m0 + rows - 1.
template <int L, int R>
__device__ __forceinline__ void gemm_rows(const TileRegs& T, const uint16_t* __restrict__ x,
                                          int64_t K, int64_t m0, int rows, int col0, int lane,
                                          int64_t tile, int64_t N, float g,
                                          uint16_t* __restrict__ y) {
  uint4 xr[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) load_x_bf16(x, K, m0 + r, col0, xr[r]);
    else for (int j = 0; j < 4; ++j) xr[r][j] = make_uint4(0, 0, 0, 0);
  }
  float part[R][8];
  tile_dot_bf16<R>(T, xr, part);
  gemm_write<L, R>(part, m0, rows, lane, tile, N, g, y);
}

// The first batch (rows 0 .. rows - 1) with the tile: the rows' loads go out
// first (a padding row's are skipped under a branch of the whole wave; they
// all precede the tile's, so the waits for the tile stay exact), then the
// tile's, and each slab is multiplied as it lands. T keeps the tile.
template <int L, int R>
__device__ __forceinline__ void gemm_first(const uint8_t* __restrict__ tile_ptr,
                                           const uint16_t* __restrict__ x, int64_t K, int rows,
                                           int col0, int lane, int64_t tile, int64_t N, float g,
                                           uint16_t* __restrict__ y, TileRegs& T) {
  uint4 xr[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) load_x_bf16(x, K, r, col0, xr[r]);
    else for (int j = 0; j < 4; ++j) xr[r][j] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_tile_scales_first(tile_ptr, lane, T);
  __builtin_amdgcn_sched_barrier(0);
  float part[R][8];
  tile_dot_bf16<R>(T, xr, part);
  gemm_write<L, R>(part, 0, rows, lane, tile, N, g, y);
}

// Q panels: the row block's tiles streamed in turn for rows m0 .. m0 + rows - 1.
template <int L, int R>
__device__ __forceinline__ void gemm_rows_panels(const uint8_t* __restrict__ blk_tiles, int64_t Q,
                                                 const uint16_t* __restrict__ x, int64_t K,
                                                 int64_t m0, int rows, int col0, int lane,
                                                 int64_t blk, int64_t N, float g,
                                                 uint16_t* __restrict__ y) {
  float acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[r][i] = 0.0f;
#pragma unroll 1
  for (int64_t q = 0; q < Q; ++q) {
    uint4 xr[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows) load_x_bf16(x, K, m0 + r, q * (L * 32) + col0, xr[r]);
      else for (int j = 0; j < 4; ++j) xr[r][j] = make_uint4(0, 0, 0, 0);
    }
    TileRegs T;
    load_tile(blk_tiles + q * kTileBytes, lane, T);
    tile_dot_bf16<R, true>(T, xr, acc);
  }
  gemm_write<L, R>(acc, m0, rows, lane, blk, N, g, y);
}

// L = Kp / 32 of the matrix's panel width; K = Q Kp. The host passes the
// row-block count nrb, Q and the tensor scale's address: computed here, their
// 64-bit divisions by runtime values came before the first load.
template <int L>
__global__ void __launch_bounds__(256) skinny_gemm_kernel(const uint16_t* __restrict__ x,
                                                          int64_t M, int64_t K,
                                                          const uint8_t* __restrict__ w,
                                                          int64_t N, uint16_t* __restrict__ y,
                                                          int64_t nrb, int64_t Q,
                                                          const float* __restrict__ gp) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row block of W
  if (blk >= nrb) return;
  const float g = gp[0];
  if (Q > 1) {
    const uint8_t* tiles = w + blk * Q * kTileBytes;
    const int col0 = 32 * (lane % L);
#pragma unroll 1
    for (int64_t m0 = 0; m0 < M; m0 += 8) {
      const int rows = (int)((M - m0) < 8 ? (M - m0) : 8);
      if (rows > 4)
        gemm_rows_panels<L, 8>(tiles, Q, x, K, m0, rows, col0, lane, blk, N, g, y);
      else if (rows > 2)
        gemm_rows_panels<L, 4>(tiles, Q, x, K, m0, rows, col0, lane, blk, N, g, y);
      else if (rows > 1)
        gemm_rows_panels<L, 2>(tiles, Q, x, K, m0, rows, col0, lane, blk, N, g, y);
      else
        gemm_rows_panels<L, 1>(tiles, Q, x, K, m0, rows, col0, lane, blk, N, g, y);
    }
    return;
  }
  const int64_t tile = blk;
  TileRegs T;
  const int col0 = 32 * (lane % L);
  // the first batch's rows are requested before the tile, so each slab is
  // multiplied as it lands (the later batches reuse the tile in registers)
  {
    const int rows = (int)(M < 8 ? M : 8);
    if (rows > 4)
      gemm_first<L, 8>(w + tile * kTileBytes, x, K, rows, col0, lane, tile, N, g, y, T);
    else if (rows > 2)
      gemm_first<L, 4>(w + tile * kTileBytes, x, K, rows, col0, lane, tile, N, g, y, T);
    else if (rows > 1)
      gemm_first<L, 2>(w + tile * kTileBytes, x, K, rows, col0, lane, tile, N, g, y, T);
    else
      gemm_first<L, 1>(w + tile * kTileBytes, x, K, rows, col0, lane, tile, N, g, y, T);
  }
#pragma unroll 1
  for (int64_t m0 = 8; m0 < M; m0 += 8) {
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


// ---- MFMA variant for K = 2048 -----------------------------------------------------------
//
// Four waves per block, each taking 16 rows of W at a time (packed tiles 2b
// and 2b + 1, 8 rows each) in a grid-stride loop; the rows of x, 16 at a time,
// are the MFMA's columns. The weights are decoded exactly to BF16 (dense.hpp)
// once per 16 rows of x, about 2 VALU instructions per weight, where the VALU
// product spends 0.5 + 0.5 M. The 16 rows of x are staged once per block in
// LDS (16-byte piece p of row r stored at piece p ^ (r % 16), so the 16 rows'
// same piece fall in 16 different bank groups): every wave reads its B
// operands there instead of from L2, which at M = 6 would move more bytes
// than W itself.
// Lane l holds W row l % 16 (chunk 4q + l / 16) and x row l % 16; D row
// 4 (l / 16) + r is W row 16 b + 4 (l / 16) + r.
constexpr int kGemmDenseMinRows = 4;
constexpr int kGemmXStride = 4096;  // bytes per staged row of x
constexpr int kGemmDenseWaves = 4;
// grid-stride beyond: 512 blocks of four waves is what is resident at two waves
// per SIMD (the kernel's registers); 1024 ran in two generations (248K head
// 74.3 us against 73.1), 768 in one and a half (83.6 us)
constexpr int64_t kGemmDenseMaxBlocks = 512;

// The chunks of 16-row block blk of W in MFMA order (zeros past the last tile
// or block).
__device__ __forceinline__ void load_gemm_block(const uint8_t* __restrict__ w, int64_t ntiles,
                                                int64_t blk, int m, int grp, DenseRows<16>& d) {
  const int64_t t = 2 * blk + (m >> 3);  // this lane's tile
  const bool valid = t < ntiles;
  const uint8_t* tile = w + (valid ? t : ntiles - 1) * kTileBytes;  // always issued
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    uint4 c;
    uint32_t sc;
    load_dense_chunk(tile, 64, m & 7, 4 * q + grp, c, sc);
    d.c[q] = valid ? c : make_uint4(0, 0, 0, 0);
    d.s[q] = valid ? sc : 0u;
  }
}

__global__ void __launch_bounds__(64 * kGemmDenseWaves) skinny_gemm_dense_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint8_t* __restrict__ w, int64_t N,
    uint16_t* __restrict__ y) {
  constexpr int64_t K = 2048;
  extern __shared__ __align__(16) uint8_t xs[];  // [rows][256 pieces of 16 bytes]
  const int lane = threadIdx.x & 63, m = lane & 15, grp = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int64_t ntiles = tiles_per_matrix(N, K);
  const int64_t nblk = (ntiles + 1) / 2;  // 16-row blocks of W
  const float g = reinterpret_cast<const float*>(w + gscale_offset(1, N, K))[0];
#pragma unroll 1
  for (int64_t c0 = 0; c0 < M; c0 += 16) {
    const int rows = (M - c0) < 16 ? (int)(M - c0) : 16;
    __syncthreads();  // the previous rows' reads are done
    for (int i = threadIdx.x; i < rows * 256; i += 64 * kGemmDenseWaves) {
      const int r = i >> 8, c = i & 255;  // 256 pieces of 16 bytes per row
      *reinterpret_cast<uint4*>(xs + r * kGemmXStride + 16 * (c ^ (r & 15))) =
          reinterpret_cast<const uint4*>(x + (c0 + r) * K)[c];
    }
    __syncthreads();
    const bool valid = m < rows;
    const uint8_t* xrow = xs + m * kGemmXStride;
#pragma unroll 1
    for (int64_t blk = (int64_t)blockIdx.x * kGemmDenseWaves + wave; blk < nblk;
         blk += (int64_t)gridDim.x * kGemmDenseWaves) {
      DenseRows<16> d;
      load_gemm_block(w, ntiles, blk, m, grp, d);
      f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        bf16x8 a[4];
        dense_a<16>(d, q, a);
        uint4 xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xv[e] = valid ? *reinterpret_cast<const uint4*>(
                              xrow + 16 * ((4 * (4 * q + grp) + e) ^ m))
                        : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_bf16(a[e], as_bf16x8(xv[e]), acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (valid) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t n = 16 * blk + 4 * grp + r;
          if (n < N) y[(c0 + m) * N + n] = f32_to_bf16_rne(acc[r] * g);
        }
      }
    }
  }
}

// ---- MFMA, K split over the four waves (K = 2048, 4 <= M <= 16, few rows of W) -----------
//
// With few 16-row blocks of W (N = 64: four) the kernel above runs one block
// whose waves each decode a whole 16 x 2048 block after staging x: three
// round trips and the full decode in a row, about 10 us for 74 KB. Here a
// block takes one 16-row block of W and its four waves split K in quarters
// (chunk columns 4 w .. 4 w + 3): each lane requests its W chunks and its x
// pieces together (x straight from L2: 1 KB per row and wave), decodes a
// quarter of the block, and the four partial D tiles are added in LDS in wave
// order.
constexpr int64_t kGemmSplitKMaxBlocks = 256;  // 16-row blocks of W (N <= 4096)

// One 16-row block blk of W, K split over waves 0-3 of the calling block (any
// further waves only join the barrier; every wave of the block must call it).
__device__ __forceinline__ void splitk_block(const uint16_t* __restrict__ x, int64_t M,
                                             const uint8_t* __restrict__ w, int64_t N,
                                             uint16_t* __restrict__ y, int64_t blk,
                                             f32x4 (*part)[64]) {
  constexpr int64_t K = 2048;
  const int lane = threadIdx.x & 63, m = lane & 15, grp = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int64_t ntiles = tiles_per_matrix(N, K);
  const int64_t t = 2 * blk + (m >> 3);  // this lane's tile
  const bool valid = m < M;
  const float g = reinterpret_cast<const float*>(w + gscale_offset(1, N, K))[0];
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (wave < kGemmDenseWaves) {
    DenseRows<4> d;
    // every load is issued (past the last tile or row: the last one, zeroed
    // after the load), so the compiler counts the loads in flight exactly
    const bool tvalid = t < ntiles;
    const uint8_t* tile = w + (tvalid ? t : ntiles - 1) * kTileBytes;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int q = 4 * wave + qq;
      uint4 c;
      uint32_t sc;
      load_dense_chunk(tile, 64, m & 7, 4 * q + grp, c, sc);
      d.c[qq] = tvalid ? c : make_uint4(0, 0, 0, 0);
      d.s[qq] = tvalid ? sc : 0u;
    }
    // x row m, pieces 4 (4 q + grp) + e of 16 bytes (8 BF16), q in this wave's
    // quarter; a lane past the last row reads row M - 1 (its D column, the
    // only one its operand reaches, is not written), so no load is behind a
    // branch
    uint4 xv[4][4];
    const uint4* xrow = reinterpret_cast<const uint4*>(x + (valid ? m : M - 1) * K);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[qq][e] = xrow[4 * (4 * (4 * wave + qq) + grp) + e];
    __builtin_amdgcn_sched_barrier(0);  // every load out before the first product
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      bf16x8 a[4];
      dense_a<4>(d, qq, a);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_bf16(a[e], as_bf16x8(xv[qq][e]), acc);
    }
    if (wave > 0) part[wave - 1][lane] = acc;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int v = 0; v < kGemmDenseWaves - 1; ++v) {
      const f32x4 o = part[v][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += o[r];
    }
    if (valid) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = 16 * blk + 4 * grp + r;
        if (n < N) y[m * N + n] = f32_to_bf16_rne(acc[r] * g);
      }
    }
  }
}

__global__ void __launch_bounds__(64 * kGemmDenseWaves) skinny_gemm_splitk_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint8_t* __restrict__ w, int64_t N,
    uint16_t* __restrict__ y) {
  __shared__ f32x4 part[kGemmDenseWaves - 1][64];
  splitk_block(x, M, w, N, y, blockIdx.x, part);
}

}  // namespace nvfp4moe
