// common.hpp - packed NVFP4 geometry and wavefront building blocks for gfx950.
//
// Packed layout of one [N][K] matrix (K = 32 * 2^j <= 2048):
//   chunk     16 bytes of codes = 32 consecutive elements of one row
//   L         chunks per row = K / 32 (lanes that share a row in a slab)
//   slab      64 consecutive chunks in canonical row-major order = 1 KB, one
//             128-bit load per lane of a wave64
//   tile      8 slabs = 16384 / K rows: 8 KB of codes followed by 1 KB of
//             scales, scales arranged [lane][slab][2] so that one 128-bit
//             load gives a lane the two E4M3 scales of each of its 8 chunks
//   matrix    ceil(N / rows_per_tile) tiles (rows past N are zero)
//   tensor    G matrices back to back, then the G FP32 tensor scales
// Lane l of slab i of tile t holds chunk 64 i + l of the tile: row
// t * rows_per_tile + i * (64 / L) + l / L, elements 32 (l % L) ... + 31.
// A lane therefore sees the same 32 columns in every slab, so activation
// values stay in its registers for a whole tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4moe {

constexpr int kWave = 64;
constexpr int kSlabsPerTile = 8;
constexpr int kTileCodeBytes = 8192;
constexpr int kTileBytes = 9216;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int64_t rows_per_tile(int64_t K) { return 16384 / K; }
__host__ __device__ constexpr int64_t tiles_per_matrix(int64_t N, int64_t K) {
  return (N + rows_per_tile(K) - 1) / rows_per_tile(K);
}
__host__ __device__ constexpr int64_t matrix_bytes(int64_t N, int64_t K) {
  return tiles_per_matrix(N, K) * kTileBytes;
}
__host__ __device__ constexpr int64_t gscale_offset(int64_t G, int64_t N, int64_t K) {
  return G * matrix_bytes(N, K);
}

// ---- element and scale decode (one instruction per pair / per scale) ----------

// Two E2M1 codes (byte `sel` of w: low nibble first) -> two BF16, exact.
__device__ __forceinline__ bf16x2 fp4_pair_bf16(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  }
}

// Two E2M1 codes -> two FP32, exact.
__device__ __forceinline__ f32x2 fp4_pair_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// E4M3 code in byte `sel` of w -> FP32, exact (gfx950 FP8 is the OCP format).
__device__ __forceinline__ float e4m3_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
  }
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Scale of half h (0: elements 0-15, 1: 16-31) of slab i from a lane's 16 scale bytes.
__device__ __forceinline__ float tile_scale(const uint4& sv, int i, int h) {
  const int byte = 2 * i + h;
  return e4m3_f32(u4_get(sv, byte >> 2), byte & 3);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// 128-bit load that is not kept in the caches longer than needed: weights are
// read once per step.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---- cross-lane exchange ------------------------------------------------------------

__device__ __forceinline__ float xor_shuffle(float v, int d) { return __shfl_xor(v, d, 64); }

// Segmented reduction of per-slab partial sums over the L lanes that share a
// row. In: v[8] per lane (slab 0..7). Out: v[0 .. 8/min(L,8)) hold full sums;
// value j of lane l belongs to slab reduced_slab<L>(l) + j. Halving exchanges
// first (each lane keeps half of its values and receives the partner's
// matching half), then plain butterflies once one value is left.
template <int L>
__device__ __forceinline__ void reduce_slabs(float (&v)[8], int lane) {
  constexpr int kHalvings = (L >= 8) ? 3 : (L == 4 ? 2 : (L == 2 ? 1 : 0));
  int count = 8;
#pragma unroll
  for (int t = 0; t < kHalvings; ++t) {
    const int d = L >> (t + 1);
    const bool upper = (lane & d) != 0;
    const int half = count >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < half) {
        const float a = v[j], b = v[j + half];
        const float send = upper ? a : b;
        const float keep = upper ? b : a;
        v[j] = keep + xor_shuffle(send, d);
      }
    }
    count = half;
  }
#pragma unroll
  for (int d = (L >= 8 ? L / 16 : 0); d >= 1; d >>= 1) v[0] += xor_shuffle(v[0], d);
}

template <int L>
__device__ __forceinline__ int reduced_slab(int lane) {
  if constexpr (L >= 8) {
    constexpr int shift = (L == 8) ? 0 : (L == 16 ? 1 : (L == 32 ? 2 : 3));
    return ((lane & (L - 1)) >> shift) & 7;
  } else {
    constexpr int shift = (L == 4) ? 1 : (L == 2 ? 2 : 3);
    return (lane & (L - 1)) << shift;
  }
}

// Lanes that write a reduced value (one per distinct result).
template <int L>
__device__ __forceinline__ bool reduced_writer(int lane) {
  if constexpr (L > 8) return (lane & (L / 8 - 1)) == 0;
  return true;
}

template <int L>
constexpr int reduced_count() {
  return L >= 8 ? 1 : 8 / L;
}

// Row of a tile held by (slab i, lane l).
template <int L>
__device__ __forceinline__ int tile_row(int slab, int lane) {
  return slab * (64 / L) + lane / L;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace nvfp4moe
