// router.hpp - router projection in front of top-k routing: logits = x W_r^T
// with BF16 rows x [M][H], a BF16 router matrix W_r [E][H] and FP32 sums and
// output (the routed mixture-of-experts model of the Elsa page, "The card and
// the model"; the router is neither an NVFP4 expert nor an FP8 projection, so
// it stays BF16).
//
// One block of four waves per expert row e: thread t owns columns
// t CPL .. t CPL + CPL - 1 (CPL = H / 256), so the block reads W_r's row once,
// coalesced, and keeps it in registers while the rows of x pass in batches of
// eight. Each wave reduces its eight partial sums over its lanes (halving
// exchanges), the four wave results add up through LDS in wave order.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

constexpr int kRouterBatch = 8;

// CPL BF16 values from p (CPL * 2 bytes, aligned to min(16, CPL * 2)).
template <int CPL>
__device__ __forceinline__ void load_bf16_run(const uint16_t* p, bool stream,
                                              uint32_t (&v)[CPL / 2]) {
  if constexpr (CPL >= 8) {
#pragma unroll
    for (int q = 0; q < CPL / 8; ++q) {
      const uint4* a = reinterpret_cast<const uint4*>(p) + q;
      const uint4 u = stream ? load_stream(a) : *a;
      v[4 * q] = u.x;
      v[4 * q + 1] = u.y;
      v[4 * q + 2] = u.z;
      v[4 * q + 3] = u.w;
    }
  } else if constexpr (CPL == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = u.x;
    v[1] = u.y;
  } else {
    v[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

template <int CPL>
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                            int64_t M,
                                                            const uint16_t* __restrict__ wr,
                                                            int E, float* __restrict__ logits) {
  constexpr int H = 256 * CPL;
  const int e = blockIdx.x;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  __shared__ float red[4][kRouterBatch];
  uint32_t wv[CPL / 2];
  load_bf16_run<CPL>(wr + (int64_t)e * H + t * CPL, true, wv);
#pragma unroll 1
  for (int64_t m0 = 0; m0 < M; m0 += kRouterBatch) {
    float part[8];
#pragma unroll
    for (int r = 0; r < kRouterBatch; ++r) {
      uint32_t xv[CPL / 2];
      if (m0 + r < M) {
        load_bf16_run<CPL>(x + (m0 + r) * H + t * CPL, false, xv);
      } else {
#pragma unroll
        for (int i = 0; i < CPL / 2; ++i) xv[i] = 0u;
      }
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL / 2; ++i)
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xv[i]), as_bf16x2(wv[i]), a, false);
      part[r] = a;
    }
    reduce_rows64<kRouterBatch>(part, lane);  // lane l: row l >> 3
    if ((lane & 7) == 0) red[wave][lane >> 3] = part[0];
    __syncthreads();
    if (t < kRouterBatch && m0 + t < M)
      logits[(m0 + t) * E + e] = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    __syncthreads();  // red is rewritten by the next batch
  }
}

}  // namespace nvfp4moe
