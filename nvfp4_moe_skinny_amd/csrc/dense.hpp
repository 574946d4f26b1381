// dense.hpp - BF16 MFMA products for expert slots with many rows.
//
// v_mfma_f32_16x16x32_bf16 multiplies a 16 x 32 block A by a 32 x 16 block B:
// lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16]
// (e = 0..7) and receives D[4 (l / 16) + r][l % 16] (r = 0..3). Which 32
// values of k one instruction covers is free as long as A and B agree: lane
// group g = l / 16 loads chunk 4q + g (32 consecutive k) of its row, and
// instruction (q, e) takes elements 8e .. 8e + 7 of every group's chunk.
//
// Weights: a code times its E4M3 scale is exact in BF16 (an E2M1 value has at
// most 2 significant bits, an E4M3 value 4, BF16 holds 8). It is formed as
// FP32 code x FP32 scale, then rounded to BF16, which changes nothing. (The
// conversion instruction's own scale operand applies only the power-of-two
// part of a scale, so it cannot carry an E4M3 scale.) The tensor scale g is
// applied to the FP32 result.
// Activations: BF16 rows as stored. h (FP32) enters as hi + lo, both BF16
// (hi = RNE(h), lo = RNE(h - hi)): 16 significant bits, a relative error of at
// most 2^-17 per element, two MFMAs per block.
//
// The loads read a tile of the packed layout in its own order: lane l takes
// chunk 4q + l / 16 of row l % 16 (16 bytes of codes, two scale bytes) for
// each q, so 16 lanes cover one chunk column of 16 rows.
#pragma once

#include "tile.hpp"

namespace nvfp4moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Slots with at least this many rows take the MFMA path by default, by the
// number of rows M of the step (crossovers measured on the MoE decode step,
// H = 2048, I = 512, E = 256, top-8, uniform and Zipf(1.1) routing): with one
// row per VALU batch (9 <= M <= 16) a slot of 3 rows is already cheaper on
// MFMA, whose cost hardly depends on the row count up to 16, and such slots
// were the launch's last items (M = 16: 51.9 -> 46.8 us, M = 12: 52.6 ->
// 36.6 us against a threshold of 16); with RMAX-row batches the VALU path
// holds out longer (M <= 32: 6, above: 8). M <= 8 keeps every slot on VALU,
// as the two-launch schedule needs. moe_nvfp4_route_decode keeps 16.
inline int dense_rows_default(int64_t M, bool routed) {
  if (!routed || M <= 8) return 16;
  if (M <= 16) return 3;
  return M <= 32 ? 6 : 8;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 codes (one word, element 0 in the low nibble) times scale s -> 8 BF16.
__device__ __forceinline__ bf16x8 decode8_bf16(uint32_t w, float s) {
  const f32x2 a = fp4_pair_f32(w, 0), b = fp4_pair_f32(w, 1);
  const f32x2 c = fp4_pair_f32(w, 2), d = fp4_pair_f32(w, 3);
  bf16x8 r;
  r[0] = (__bf16)(a[0] * s);
  r[1] = (__bf16)(a[1] * s);
  r[2] = (__bf16)(b[0] * s);
  r[3] = (__bf16)(b[1] * s);
  r[4] = (__bf16)(c[0] * s);
  r[5] = (__bf16)(c[1] * s);
  r[6] = (__bf16)(d[0] * s);
  r[7] = (__bf16)(d[1] * s);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// h as one 32-bit word: BF16 hi in the low half, BF16 lo in the high half.
__device__ __forceinline__ uint32_t pack_hilo(float h) {
  const uint16_t hi = f32_to_bf16_rne(h);
  const uint16_t lo = f32_to_bf16_rne(h - bf16_to_f32(hi));
  return (uint32_t)hi | ((uint32_t)lo << 16);
}

// Eight packed words -> the hi and lo BF16 operands.
__device__ __forceinline__ void split_hilo(const uint4& w0, const uint4& w1, bf16x8& hi, bf16x8& lo) {
  const uint4 h = make_uint4((w0.x & 0xFFFFu) | (w0.y << 16), (w0.z & 0xFFFFu) | (w0.w << 16),
                             (w1.x & 0xFFFFu) | (w1.y << 16), (w1.z & 0xFFFFu) | (w1.w << 16));
  const uint4 l = make_uint4((w0.x >> 16) | (w0.y & 0xFFFF0000u), (w0.z >> 16) | (w0.w & 0xFFFF0000u),
                             (w1.x >> 16) | (w1.y & 0xFFFF0000u), (w1.z >> 16) | (w1.w & 0xFFFF0000u));
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// Codes and scales of NQ chunk columns of one 16-row block, in MFMA order.
template <int NQ>
struct DenseRows {
  uint4 c[NQ];
  uint32_t s[NQ];  // two E4M3 bytes: elements 0-15, 16-31 of the chunk
};

// Row n (< rows_per_tile) of a packed tile, chunk c: codes and scale bytes.
// L = K / 32 chunks per row; a slab holds 64 / L rows.
__device__ __forceinline__ void load_dense_chunk(const uint8_t* tile, int L, int n, int c,
                                                 uint4& code, uint32_t& scales) {
  const int rps = 64 / L;
  const int slab = n / rps;
  const int pos = (n % rps) * L + c;  // lane position within the slab
  code = load_stream(reinterpret_cast<const uint4*>(tile + slab * 1024) + pos);
  scales = *reinterpret_cast<const uint16_t*>(tile + kTileCodeBytes + pos * 16 + slab * 2);
}

// Hides the registers from the optimiser (no instruction): called once per
// pass over column blocks, it keeps the decode of every chunk column from
// being hoisted out of the pass loop (which would hold 4 NQ decoded operands).
template <int NQ>
__device__ __forceinline__ void opaque_dense(DenseRows<NQ>& d) {
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    asm volatile("" : "+v"(d.c[q].x), "+v"(d.c[q].y), "+v"(d.c[q].z), "+v"(d.c[q].w),
                 "+v"(d.s[q]));
}

// A operands of chunk column q: elements 8e .. 8e + 7 for e = 0..3.
template <int NQ>
__device__ __forceinline__ void dense_a(const DenseRows<NQ>& d, int q, bf16x8 (&a)[4]) {
  const float s0 = e4m3_f32(d.s[q], 0), s1 = e4m3_f32(d.s[q], 1);
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = decode8_bf16(u4_get(d.c[q], e), e < 2 ? s0 : s1);
}

}  // namespace nvfp4moe
