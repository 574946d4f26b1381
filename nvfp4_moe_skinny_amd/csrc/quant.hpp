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
// (16 correctly rounded quotients per block) and keeps one block per thread.
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
  // four chunks a thread in flight (one at a time: 191.4 us for the
  // [256][1024][2048] pass, four: 181.7 us, eight: 185.2 us); past the end a
  // thread reads its first chunk of the step again (a repeat leaves the
  // maximum unchanged)
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; c0 < chunks;
       c0 += 4 * stride) {
    uint4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + u * stride < chunks ? c0 + u * stride : c0;
      a[u] = load_stream(xm + 2 * c);
      b[u] = load_stream(xm + 2 * c + 1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[8] = {a[u].x, a[u].y, a[u].z, a[u].w, b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
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

// The two BF16 elements of word w (low half first) divided by sg, each
// quotient correctly rounded (q0 = RN(x y), then one FMA correction with the
// exact remainder; y = RN(1 / sg)), converted to E2M1 codes into byte SEL of
// `codes`. The correction turns -0 into +0 (+0 + -0 rounds to +0), so the
// quotient takes x's sign back (a no-op for every other value).
template <int SEL>
__device__ __forceinline__ uint32_t quotients_to_e2m1(uint32_t codes, uint32_t w, float y,
                                                     float sg) {
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
  const float q0 = __fmul_rn(x0, y), q1 = __fmul_rn(x1, y);
  const float r0 =
      __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, sg, x0), y, q0), x0);
  const float r1 =
      __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q1, sg, x1), y, q1), x1);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, r0, r1, 1.0f, SEL);
}

// One 16-element block i (of matrix gi) per thread.
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, int64_t i,
                                            int64_t gi, const uint32_t* __restrict__ amax,
                                            uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales) {
  const uint4* xp = reinterpret_cast<const uint4*>(x) + 2 * i;
  const uint4 a = load_stream(xp), b = load_stream(xp + 1);
  const float gv = quant_g(amax[gi]);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t mb = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) mb = max(mb, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  const float t = __fdiv_rn(__uint_as_float(mb << 16), __fmul_rn(6.0f, gv));
  const uint32_t sc = e4m3_rne_code(t);
  const float sg = __fmul_rn(e4m3_f32(sc, 0), gv);
  // The 16 quotients |x| / sg, each correctly rounded, with one division:
  // Markstein's method. With y the correctly rounded reciprocal of sg and
  // q0 = RN(|x| y) (within one ulp of the quotient), the remainder
  // |x| - q0 sg is exact in one FMA and RN(q0 + remainder * y) is the
  // correctly rounded quotient, provided nothing leaves the normal range. So
  // the fast form is taken for 2^-100 <= sg <= 2^100 (y and the quotients near
  // E2M1's decision points, all >= 0.25, normal; smaller quotients round to
  // code 0 either way, and the block scale keeps the quotients below 12), and
  // the division itself otherwise (sg zero, subnormal, huge, inf or NaN).
  // In the fast form the signed quotients go to the E2M1 conversion
  // instruction, two per instruction: it rounds to nearest even on the E2M1
  // grid and saturates at 6 exactly as e2m1_rne_code does for every finite
  // value (checked on the chip over every decision point and its neighbours);
  // it differs only for NaN, which the fast form never sees (a NaN or inf
  // element makes the matrix maximum, hence sg, NaN or inf).
  const bool fast = sg >= 0x1p-100f && sg <= 0x1p100f;
  uint32_t q[2] = {0u, 0u};
  if (fast) {
    const float y = __fdiv_rn(1.0f, sg);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      q[h] = quotients_to_e2m1<0>(q[h], w[4 * h], y, sg);
      q[h] = quotients_to_e2m1<1>(q[h], w[4 * h + 1], y, sg);
      q[h] = quotients_to_e2m1<2>(q[h], w[4 * h + 2], y, sg);
      q[h] = quotients_to_e2m1<3>(q[h], w[4 * h + 3], y, sg);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t bits = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t mag = sg > 0.0f ? e2m1_rne_code(__fdiv_rn(bf16_abs_f32(bits), sg)) : 0u;
      q[j >> 3] |= (((bits >> 15) << 3) | mag) << (4 * (j & 7));
    }
  }
  *reinterpret_cast<uint2*>(codes + 8 * i) = make_uint2(q[0], q[1]);
  scales[i] = (uint8_t)sc;
}

// Grid (blocks of the matrix / kQuantThreads, G): the matrix is the
// workgroup's row, so no thread divides its block index (a 64-bit division
// ahead of every load: 254.6 -> 236.8 us for [256][1024][2048]).
__global__ void __launch_bounds__(kQuantThreads) quant_blocks_kernel(
    const uint16_t* __restrict__ x, int64_t blocks_per_matrix,
    const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t il = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  const int64_t gi = blockIdx.y;
  if (il < blocks_per_matrix)
    quant_block(x, gi * blocks_per_matrix + il, gi, amax, codes, scales);
}

// g[i] = amax / 2688 (1 if 0), in place over the maxima.
__global__ void __launch_bounds__(kQuantThreads) quant_finish_kernel(float* __restrict__ g,
                                                                     int64_t G) {
  const int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i < G) g[i] = quant_g(__float_as_uint(g[i]));
}

}  // namespace nvfp4moe
