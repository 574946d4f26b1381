// fp8.hpp - skinny product of BF16 rows with an FP8 E4M3 matrix that carries
// one FP32 scale for the whole tensor: y = (x W^T) * s, FP32 sums, BF16 out.
//
// W is [N][K] bytes, row-major, exactly as stored: FP8 needs no repacking,
// since a 16-byte chunk of a row is already 16 whole elements. K is 1024,
// 2048 or 4096, so a row is S = K / 1024 slabs of 1 KB.
// One wave owns a tile of 8 slabs (8 KB, 8 / S rows) and loads it with eight
// 128-bit loads per lane: lane l takes bytes 16 l .. 16 l + 15 of each slab,
// so it sees the same 16 columns of each of the row's S slabs and its
// activation values stay in registers for the whole tile.
// Decode: v_cvt_scalef32_pk_bf16_fp8 (two elements per instruction, exact:
// E4M3 has 4 significant bits), then v_dot2c_f32_bf16 against the activation
// pairs; the tensor scale multiplies the reduced FP32 sum once.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

constexpr int kFp8SlabBytes = 1024;
constexpr int kFp8TileBytes = 8 * kFp8SlabBytes;

// Two E4M3 elements (bytes 2 hi_word, 2 hi_word + 1 of w) -> two BF16, exact.
__device__ __forceinline__ bf16x2 fp8_pair_bf16(uint32_t w, bool hi_word) {
  return hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

// The lane's 16 columns of each of the S slab positions of x rows m0 ..
// m0 + R - 1 (rows past M read row M - 1).
template <int R, int S>
__device__ __forceinline__ void load_fp8_rows(const uint16_t* __restrict__ x, int64_t m0,
                                              int64_t M, int lane, uint4 (&xr)[R][S][2]) {
  constexpr int K = S * kFp8SlabBytes;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = m0 + r < M ? m0 + r : M - 1;
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const uint4* p = reinterpret_cast<const uint4*>(x + row * K + q * 1024 + 16 * lane);
      xr[r][q][0] = p[0];
      xr[r][q][1] = p[1];
    }
  }
}

// One wave per tile of 8 / S rows; rows of x in batches of up to R.
template <int S, int RMAX>
__global__ void __launch_bounds__(64) fp8_skinny_gemm_kernel(const uint16_t* __restrict__ x,
                                                            int64_t M,
                                                            const uint8_t* __restrict__ w,
                                                            const float* __restrict__ scale,
                                                            int64_t N, uint16_t* __restrict__ y) {
  constexpr int RPT = 8 / S;  // rows per tile
  constexpr int K = S * kFp8SlabBytes;
  const int lane = threadIdx.x;
  const int64_t tile = xcd_block((int)blockIdx.x, (int)gridDim.x);
  const int64_t n0 = tile * RPT;
  const float s = scale[0];
  const int rlane = lane >> (6 - (RPT == 8 ? 3 : RPT == 4 ? 2 : RPT == 2 ? 1 : 0));
  // The first batch's activation rows are requested before the tile, so each
  // slab is multiplied as it lands. Every load is issued (a row past M or N
  // reads the last one: its results are not written), since a load skipped
  // under a branch makes the compiler's waits cover later loads too.
  uint4 xr[RMAX][S][2];
  load_fp8_rows<RMAX, S>(x, 0, M, lane, xr);
  __builtin_amdgcn_sched_barrier(0);
  // codes: slab i is row i / S, columns (i % S) * 1024 + 16 lane .. + 15
  uint4 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0 + i / S < N ? n0 + i / S : N - 1;
    c[i] = load_stream(reinterpret_cast<const uint4*>(w + n * K + (i % S) * 1024) + lane);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
  for (int64_t m0 = 0; m0 < M; m0 += RMAX) {
    if (m0 > 0) load_fp8_rows<RMAX, S>(x, m0, M, lane, xr);
    float part[RMAX][8];
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) part[r][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x2 wv[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) wv[p] = fp8_pair_bf16(u4_get(c[i], p >> 1), (p & 1) != 0);
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        float a = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p)
          a = __builtin_amdgcn_fdot2_f32_bf16(wv[p], as_bf16x2(u4_get(xr[r][i % S][p >> 2], p & 3)),
                                               a, false);
        part[r][i / S] += a;  // slabs of one row add up in slab order
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      reduce_rows64<RPT>(part[r], lane);
      const int64_t n = n0 + rlane;
      const bool writer = (lane & ((64 / RPT) - 1)) == 0;
      if (writer && m0 + r < M && n < N) y[(m0 + r) * N + n] = f32_to_bf16_rne(part[r][0] * s);
    }
  }
}

}  // namespace nvfp4moe
