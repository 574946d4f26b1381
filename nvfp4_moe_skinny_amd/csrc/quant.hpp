// quant.hpp - BF16 matrices -> canonical NVFP4 (E2M1 codes, one E4M3 scale per
// 16 elements along K, one FP32 scale per matrix) on the device.
//
// The pages name only the tool that quantized a BF16 head to NVFP4 (the
// "Files" list of the Qwen3.8-27B NVFP4 lm_head recipe page); the recipe
// here is the plain amax one, with every division and product in FP32:
//   g   = amax / 2688 over the matrix (6 * 448: the largest E2M1 magnitude
//         times the largest E4M3 value), 1 if amax = 0;
//   s_b = E4M3 round-to-nearest-even of amax_b / (6 g), saturating at 448;
//   q   = sign of x | E2M1 round-to-nearest-even of |x| / (s_b g),
//         saturating at 6; magnitude 0 where s_b g = 0.
// Passes: clear the per-matrix maxima, take them (integer maximum of the
// magnitude bits, which order like the values), quantize each block, then
// turn the maxima into g.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

constexpr int kQuantThreads = 256;
// Workgroups of the maximum pass per matrix: a pass of tens of thousands of
// short workgroups is bound by how fast they start (measured over
// [256][1024][2048]: 314 us with 256 workgroups per matrix, 184 us with 16).
// The quantising pass, one thread per 16 elements, is bound by its arithmetic
// (16 correctly rounded divisions per block) and keeps one block per thread.
constexpr int kQuantMaxBlocksPerMatrix = 16;

// Nearest finite non-negative E4M3 code to t >= 0, ties to the even code,
// 448 (0x7E) at and above 448: the FP32 significand rounded to 3 bits in the
// normal range, t * 2^9 rounded to an integer (0..8) below 2^-6.
__device__ __forceinline__ uint32_t e4m3_rne_code(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  const uint32_t b = __float_as_uint(t);
  const int e = (int)(b >> 23) - 127;
  if (e < -6) return (uint32_t)__builtin_rintf(t * 512.0f);  // 8 is 2^-6, code 0x08
  uint32_t m = (b >> 20) & 7u;
  const uint32_t rem = b & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
  const uint32_t code = ((uint32_t)(e + 7) << 3) + m;  // m = 8 carries into the exponent
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 magnitude code of v >= 0: count of midpoints of {0, .5, 1, 1.5, 2, 3,
// 4, 6} below v, a midpoint itself going to the even neighbour.
__device__ __forceinline__ uint32_t e2m1_rne_code(float v) {
  return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) +
         (uint32_t)(v >= 1.75f) + (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) +
         (uint32_t)(v > 5.0f);
}

__device__ __forceinline__ float bf16_abs_f32(uint32_t bits16) {
  return __uint_as_float((bits16 & 0x7FFFu) << 16);
}

__global__ void __launch_bounds__(kQuantThreads) quant_clear_kernel(uint32_t* __restrict__ amax,
                                                                    int64_t G) {
  const int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i < G) amax[i] = 0u;
}

// amax[g] = max |x| over matrix g (as FP32 bits); grid (blocks, G).
__global__ void __launch_bounds__(kQuantThreads) quant_amax_kernel(const uint16_t* __restrict__ x,
                                                                   int64_t chunks,
                                                                   uint32_t* __restrict__ amax) {
  const int64_t gi = blockIdx.y;
  const uint4* xm = reinterpret_cast<const uint4*>(x) + gi * chunks * 2;  // 16 BF16 per chunk
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * kQuantThreads) {
    const uint4 a = load_stream(xm + 2 * c), b = load_stream(xm + 2 * c + 1);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
  __shared__ uint32_t red[kQuantThreads / 64];
  m = wave_max_u32(m << 16);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) r = max(r, red[w]);
    atomicMax(amax + gi, r);
  }
}

__device__ __forceinline__ float quant_g(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
}

// One 16-element block (row n, block b) of matrix g per thread.
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, int64_t i,
                                            int64_t blocks_per_matrix,
                                            const uint32_t* __restrict__ amax,
                                            uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales) {
  const float gv = quant_g(amax[i / blocks_per_matrix]);
  const uint4* xp = reinterpret_cast<const uint4*>(x) + 2 * i;
  const uint4 a = load_stream(xp), b = load_stream(xp + 1);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t mb = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) mb = max(mb, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  const float t = __fdiv_rn(__uint_as_float(mb << 16), __fmul_rn(6.0f, gv));
  const uint32_t sc = e4m3_rne_code(t);
  const float sg = __fmul_rn(e4m3_f32(sc, 0), gv);
  uint32_t q[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t bits = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t mag = sg > 0.0f ? e2m1_rne_code(__fdiv_rn(bf16_abs_f32(bits), sg)) : 0u;
    q[j >> 3] |= (((bits >> 15) << 3) | mag) << (4 * (j & 7));
  }
  *reinterpret_cast<uint2*>(codes + 8 * i) = make_uint2(q[0], q[1]);
  scales[i] = (uint8_t)sc;
}

__global__ void __launch_bounds__(kQuantThreads) quant_blocks_kernel(
    const uint16_t* __restrict__ x, int64_t blocks_per_matrix, int64_t G,
    const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i < blocks_per_matrix * G) quant_block(x, i, blocks_per_matrix, amax, codes, scales);
}

// g[i] = amax / 2688 (1 if 0), in place over the maxima.
__global__ void __launch_bounds__(kQuantThreads) quant_finish_kernel(float* __restrict__ g,
                                                                     int64_t G) {
  const int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i < G) g[i] = quant_g(__float_as_uint(g[i]));
}

}  // namespace nvfp4moe
