// tile.hpp - one wavefront x one packed tile x R activation rows.
//
// A wave loads a whole tile (8 x 1 KB of codes, 1 KB of scales) with nine
// 128-bit loads per lane, keeps it in registers, and multiplies it with up
// to 8 activation rows at a time. Per slab and row a lane forms two 16-element
// partial sums (one per E4M3 block) and scales each once:
//   BF16 rows: codes -> BF16 pairs (v_cvt_scalef32_pk_bf16_fp4), then
//              v_dot2c_f32_bf16 against the BF16 activation pairs;
//   FP32 rows: codes -> FP32 pairs (v_cvt_scalef32_pk_f32_fp4), then FMA.
// E2M1 x BF16 products are exact in FP32, so only the FP32 sums round.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

struct TileRegs {
  uint4 codes[8];
  uint4 scales;
};

__device__ __forceinline__ void load_tile(const uint8_t* tile, int lane, TileRegs& t) {
  const uint4* c = reinterpret_cast<const uint4*>(tile);
#pragma unroll
  for (int i = 0; i < 8; ++i) t.codes[i] = load_stream(c + i * 64 + lane);
  t.scales = load_stream(reinterpret_cast<const uint4*>(tile + kTileCodeBytes) + lane);
}

// The same with the scale word requested first, so that slab i can be
// multiplied once the loads up to it have landed (every slab needs its scale
// bytes). Measured faster in the skinny GEMM's single-panel kernel (M = 1,
// 2048 -> 512: 3.975 -> 3.915 us) and in the M = 4 gate_up kernel once its
// activation row came in coalesced pieces ahead of the tile (14.705 -> 14.688
// us); elsewhere in the MoE kernels it measured slower (40-layer stack 1178 ->
// 1184 us).
__device__ __forceinline__ void load_tile_scales_first(const uint8_t* tile, int lane,
                                                       TileRegs& t) {
  const uint4* c = reinterpret_cast<const uint4*>(tile);
  t.scales = load_stream(reinterpret_cast<const uint4*>(tile + kTileCodeBytes) + lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) t.codes[i] = load_stream(c + i * 64 + lane);
}

// Makes the tile registers opaque to the optimiser (no instruction is
// emitted). Called at the top of every row batch, it stops the compiler from
// hoisting the decode of the whole tile out of the batch loop, which would
// keep 128-256 decoded values live and spill.
__device__ __forceinline__ void opaque_tile(TileRegs& t) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    asm volatile("" : "+v"(t.codes[i].x), "+v"(t.codes[i].y), "+v"(t.codes[i].z),
                 "+v"(t.codes[i].w));
  asm volatile("" : "+v"(t.scales.x), "+v"(t.scales.y), "+v"(t.scales.z), "+v"(t.scales.w));
}

// part[r][i] = sum over the lane's 32 columns of slab i of W * x_r (no g);
// ACC: added to part[r][i] instead (the panels of one row block).
// x[r] holds the row's 32 BF16 values of the lane's columns as 4 x uint4.
template <int R, bool ACC = false>
__device__ __forceinline__ void tile_dot_bf16(const TileRegs& t, const uint4 (&x)[R][4],
                                              float (&part)[R][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16x2 w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) w[p] = fp4_pair_bf16(u4_get(t.codes[i], p >> 2), p & 3);
    const float s0 = tile_scale(t.scales, i, 0);
    const float s1 = tile_scale(t.scales, i, 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p)
        a0 = __builtin_amdgcn_fdot2_f32_bf16(w[p], as_bf16x2(u4_get(x[r][p >> 2], p & 3)), a0,
                                             false);
#pragma unroll
      for (int p = 8; p < 16; ++p)
        a1 = __builtin_amdgcn_fdot2_f32_bf16(w[p], as_bf16x2(u4_get(x[r][p >> 2], p & 3)), a1,
                                             false);
      part[r][i] = ACC ? part[r][i] + (a0 * s0 + a1 * s1) : a0 * s0 + a1 * s1;
    }
    // keep each slab's decode next to its use (no hoisting of all decodes)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Same with FP32 activation rows: h[r] = 32 FP32 values of the lane's columns.
template <int R, bool ACC = false>
__device__ __forceinline__ void tile_dot_f32(const TileRegs& t, const float (&h)[R][32],
                                             float (&part)[R][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f32x2 w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) w[p] = fp4_pair_f32(u4_get(t.codes[i], p >> 2), p & 3);
    const float s0 = tile_scale(t.scales, i, 0);
    const float s1 = tile_scale(t.scales, i, 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        a0 = __builtin_fmaf(w[p][0], h[r][2 * p], a0);
        a0 = __builtin_fmaf(w[p][1], h[r][2 * p + 1], a0);
      }
#pragma unroll
      for (int p = 8; p < 16; ++p) {
        a1 = __builtin_fmaf(w[p][0], h[r][2 * p], a1);
        a1 = __builtin_fmaf(w[p][1], h[r][2 * p + 1], a1);
      }
      part[r][i] = ACC ? part[r][i] + (a0 * s0 + a1 * s1) : a0 * s0 + a1 * s1;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Loads the lane's 32 BF16 columns of activation row `row`. Where loads run
// ahead of their use (the MFMA column rings), callers pad a batch with a row
// that exists (results of padding rows are never written, and in these
// products no output reads another row's activations) rather than skip the
// load: a load under a branch leaves the compiler unable to count the loads
// in flight where the paths join, and its waits then also cover every load
// issued after it, prefetches included. The VALU row batches, whose products
// wait for the whole batch anyway, skip a padding row's load instead.
__device__ __forceinline__ void load_x_bf16(const uint16_t* x, int64_t ld, int64_t row, int col0,
                                            uint4 (&xr)[4]) {
  const uint4* p = reinterpret_cast<const uint4*>(x + row * ld + col0);
#pragma unroll
  for (int j = 0; j < 4; ++j) xr[j] = p[j];
}

// The lane's 32 FP32 columns of h row `row` (padding as for load_x_bf16).
__device__ __forceinline__ void load_h_f32(const float* h, int64_t ld, int64_t row, int col0,
                                           float (&hr)[32]) {
  const float4* p = reinterpret_cast<const float4*>(h + row * ld + col0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 v = p[j];
    hr[4 * j] = v.x;
    hr[4 * j + 1] = v.y;
    hr[4 * j + 2] = v.z;
    hr[4 * j + 3] = v.w;
  }
}

// A whole activation row through LDS. Loaded directly, neighbouring lanes'
// 32 columns lie 64 B (BF16) or 128 B (FP32) apart, so each 16-byte load of a
// wave touches 32 (BF16 row of 64 chunks) or 16 (FP32 row of 16 chunks)
// cache lines: 128 line requests for the row either way (4 or 8 loads).
// Requested as coalesced 1 KB pieces (8 lines each), written to the wave's own
// LDS row and read back by columns, it takes 32 (4 KB BF16 row) or 16 (2 KB
// FP32 row). load_coalesced: v[i] = src[64 i + lane].
template <int N>
__device__ __forceinline__ void load_coalesced(const uint4* src, int lane, uint4 (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = src[i * 64 + lane];
}

// Writes the N pieces to the wave's LDS row, then reads back the W 16-byte
// words of chunk c (W = 4: 32 BF16 columns; W = 8: 32 FP32 columns). Only the
// calling wave touches `lds`.
template <int N, int W>
__device__ __forceinline__ void restage_row(uint4* lds, int lane, int c, const uint4 (&v)[N],
                                            uint4 (&out)[W]) {
#pragma unroll
  for (int i = 0; i < N; ++i) lds[i * 64 + lane] = v[i];
  // other lanes' writes before this lane's reads: with no barrier here the
  // compiler may hoist a read above a write it proves is not this lane's own
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < W; ++i) out[i] = lds[W * c + i];
}

}  // namespace nvfp4moe
