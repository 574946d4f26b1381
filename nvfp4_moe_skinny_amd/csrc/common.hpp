// common.hpp - packed NVFP4 geometry and wavefront building blocks for gfx950.
//
// Packed layout of one [N][K] matrix (K % 32 == 0):
//   panel     Kp = the largest 32 * 2^j <= 2048 that divides K; the matrix's
//             columns fall into Q = K / Kp panels of Kp columns
//   chunk     16 bytes of codes = 32 consecutive elements of one row
//   L         chunks per row of a panel = Kp / 32 (lanes that share a row in
//             a slab)
//   slab      64 consecutive chunks of one panel, rows in canonical
//             row-major order = 1 KB, one 128-bit load per lane of a wave64
//   tile      8 slabs = R = 16384 / Kp rows of one panel: 8 KB of codes
//             followed by 1 KB of scales, scales arranged [lane][slab][2] so
//             that one 128-bit load gives a lane the two E4M3 scales of each
//             of its 8 chunks
//   row block R rows across the whole K: the Q tiles of its panels, back to
//             back (tile b Q + q is row block b, panel q)
//   matrix    ceil(N / R) row blocks (rows past N are zero)
//   tensor    G matrices back to back, then the G FP32 tensor scales
// Lane l of slab i of tile (b, q) holds chunk 64 i + l of the tile: row
// b R + i (64 / L) + l / L, elements q Kp + 32 (l % L) ... + 31. A lane
// therefore sees the same 32 columns in every slab of a tile, so activation
// values stay in its registers for a whole tile. When K is a power of two
// (up to 2048) there is one panel and a row block is one tile.
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

// Panel width of a K-column matrix (K % 32 == 0): the largest 32 * 2^j <= 2048
// dividing K.
__host__ __device__ constexpr int64_t panel_k(int64_t K) {
  int64_t kp = 32;
  while (kp < 2048 && K % (2 * kp) == 0) kp *= 2;
  return kp;
}
__host__ __device__ constexpr int64_t panels(int64_t K) { return K / panel_k(K); }
__host__ __device__ constexpr int64_t rows_per_tile(int64_t K) { return 16384 / panel_k(K); }
__host__ __device__ constexpr int64_t row_blocks(int64_t N, int64_t K) {
  return (N + rows_per_tile(K) - 1) / rows_per_tile(K);
}
__host__ __device__ constexpr int64_t tiles_per_matrix(int64_t N, int64_t K) {
  return row_blocks(N, K) * panels(K);
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

// Workgroups are handed to the eight XCDs (each with its own L2) in turn:
// workgroup b runs on XCD b % 8. For a grid whose size is a multiple of 8 this
// gives XCD x the consecutive logical blocks [x G / 8, (x + 1) G / 8), so the
// work items that read neighbouring bytes share an L2. Other grids keep b.
// Used where the items are uniform (the few-row MoE kernels, the FP8
// product); measured slower where a few items carry most of the work (a
// popular expert's tiles would all land on one XCD) and for the persistent
// MFMA product.
__device__ __forceinline__ int xcd_block(int b, int G) {
  if (G & 7) return b;
  return (b & 7) * (G >> 3) + (b >> 3);
}

// ---- cross-lane exchange ------------------------------------------------------------

// DPP controls (gfx9 encoding). Those named kDppXor<m> read lane l ^ m.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;  // in a 16-lane row, lane i + 8 mod 16 = i ^ 8
constexpr int kDppHalfMirror = 0x141;  // in 8 lanes, lane 7 - i = i ^ 7

__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int ctrl) {
  switch (ctrl) {
    case kDppQuadXor1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false);
    case kDppQuadXor2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false);
    case kDppRowRor4: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor4, 0xF, 0xF, false);
    case kDppHalfMirror: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor8, 0xF, 0xF, false);
  }
}

// Maximum over the wave, returned uniform: DPP within each 16-lane row, then
// the four row results through readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32(v, kDppQuadXor1));
  v = max(v, dpp_u32(v, kDppQuadXor2));
  v = max(v, dpp_u32(v, kDppRowRor4));
  v = max(v, dpp_u32(v, kDppRowRor8));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Maximum over the wave in every lane, VALU only: DPP within 16-lane rows,
// then v_permlane16_swap / v_permlane32_swap of v with itself, whose two
// results hold the partner rows' values (their maximum is the pair's).
__device__ __forceinline__ uint32_t wave_max_u32_all(uint32_t v) {
  v = max(v, dpp_u32(v, kDppQuadXor1));
  v = max(v, dpp_u32(v, kDppQuadXor2));
  v = max(v, dpp_u32(v, kDppRowRor4));
  v = max(v, dpp_u32(v, kDppRowRor8));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)b[0], (uint32_t)b[1]);
}

// The value of lane l ^ 32 (every lane of the wave active). v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with both operands v, result 1 holds the upper half's values in the
// lower lanes and result 0 the lower half's in the upper lanes.
__device__ __forceinline__ float partner32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// Halving exchange at distance d (a power of two <= 32; the whole wave
// active, d uniform): a lane whose bit log2(d) is clear returns
// a + a(partner), a lane whose bit is set b + b(partner). The partner
// differs from the lane in bit log2(d) and in no higher bit: l ^ d, except
// l ^ 7 for d = 4 (DPP has no xor-4 pattern; the half-row mirror is one).
// Instead of LDS permutes: v_permlane32_swap / v_permlane16_swap for d = 32 /
// 16 (one swap moves a's upper half and b's lower half at once) and DPP
// operands below. Both orders of the two addends give the same sum.
__device__ __forceinline__ float halve(float a, float b, int d, int lane) {
  if (d == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (d == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool upper = (lane & d) != 0;
  const float send = upper ? a : b;
  const float keep = upper ? b : a;
  const int ctrl = d == 8 ? kDppRowRor8 : (d == 4 ? kDppHalfMirror : (d == 2 ? kDppQuadXor2
                                                                           : kDppQuadXor1));
  return keep + __uint_as_float(dpp_u32(__float_as_uint(send), ctrl));
}

// v + v(partner) in every lane, same pairing as halve().
__device__ __forceinline__ float fold(float v, int d, int lane) { return halve(v, v, d, lane); }

// Sum of v[0 .. RPT) over the 64 lanes, each row separately: halving
// exchanges (a lane keeps half of its values, receives the partner's matching
// half), then plain butterflies. After: v[0] of lane l holds the full sum of
// row (l >> (6 - log2 RPT)) (all lanes of that group hold it).
template <int RPT>
__device__ __forceinline__ void reduce_rows64(float (&v)[8], int lane) {
  constexpr int kHalvings = RPT == 8 ? 3 : (RPT == 4 ? 2 : (RPT == 2 ? 1 : 0));
  int count = RPT;
#pragma unroll
  for (int t = 0; t < kHalvings; ++t) {
    const int d = 32 >> t;
    const int half = count >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < half) v[j] = halve(v[j], v[j + half], d, lane);
    }
    count = half;
  }
#pragma unroll
  for (int d = 32 >> kHalvings; d >= 1; d >>= 1) v[0] = fold(v[0], d, lane);
}

// Segmented reduction of per-slab partial sums over the L lanes that share a
// row. In: v[8] per lane (slab 0..7). Out: v[0 .. 8/min(L,8)) hold full sums;
// value j of lane l belongs to slab reduced_slab<L>(l) + j. Halving exchanges
// first (each lane keeps half of its values and receives the partner's
// matching half), then plain butterflies once one value is left; a lane's
// half is chosen by its own bit log2(d), so the partner pattern of halve()
// leaves this mapping as it is for xor partners.
template <int L>
__device__ __forceinline__ void reduce_slabs(float (&v)[8], int lane) {
  constexpr int kHalvings = (L >= 8) ? 3 : (L == 4 ? 2 : (L == 2 ? 1 : 0));
  int count = 8;
#pragma unroll
  for (int t = 0; t < kHalvings; ++t) {
    const int d = L >> (t + 1);
    const int half = count >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < half) {
        v[j] = halve(v[j], v[j + half], d, lane);
      }
    }
    count = half;
  }
#pragma unroll
  for (int d = (L >= 8 ? L / 16 : 0); d >= 1; d >>= 1) v[0] = fold(v[0], d, lane);
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
