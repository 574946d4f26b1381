// fused.hpp - routing folded into gate_up for few rows (two launches from the
// logits to the output, with token_down_combine_kernel).
//
// One block per (item, gate tile j); items are the pairs m*k + jj (row m, slot
// jj), then the shared expert's rows. Both waves of a routed item select the
// top k of row m themselves (the same per-row routine as moe_route_topk, so
// the same experts and weights bit for bit) while the row of x is already on
// its way; wave 0 then streams gate tile j of expert ids[m][jj], wave 1 the up
// tile, as in staged_gate_split_kernel. The items of tile 0 store ids and w
// for the down launch. With few rows nearly every pair has its own expert, so
// a tile per pair costs almost no extra bytes, and no grouping is needed.
#pragma once

#include "route.hpp"
#include "staged.hpp"

namespace nvfp4moe {

template <int LHC>
__global__ void __launch_bounds__(128, 4) fused_route_gate_kernel(MoeParams p,
                                                                  const float* __restrict__ logits,
                                                                  const float* __restrict__ bias,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ w) {
  constexpr int NV = LHC ? 1 : 8;  // reduced values a lane may hold
  __shared__ float up_lds[NV][64];
  __shared__ float lp[2][kRouteMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = xcd_block((int)blockIdx.x, (int)gridDim.x);
  const int item = b / p.PG, j = b % p.PG;
  const int npairs = p.M * p.k;
  const bool sh = item >= npairs;
  const int m = sh ? item - npairs : item / p.k;
  const int L = LHC ? LHC : p.LH;
  uint4 xr[1][4];
  load_x_bf16(p.x, p.H, m, 32 * (lane % L), xr[0]);
  int e = 0;
  if (!sh) {
    int my_id;
    float my_w;
    const int jj = item - m * p.k;
    // the items of tile 0 store ids and w (all k rounds, softmax); the others
    // need only the first jj + 1 experts
    route_row_core(logits, bias, p.E, p.k, m, lane, lp[wave], my_id, my_w,
                   j == 0 ? kRouteMaxK : jj + 1, j == 0);
    e = __builtin_amdgcn_readlane(my_id, jj);
    if (j == 0 && wave == 0 && lane == jj) {
      ids[item] = my_id;
      w[item] = my_w;
    }
  }
  const uint8_t* mat = sh ? p.sgu : p.gu + (int64_t)e * p.gu_mat_bytes;
  const float g = sh ? p.sgu_g[0] : p.gu_g[e];
  const int rb = wave == 0 ? j : j + p.PG;  // gate row block j, or the matching up one
  float v[8];
  if (LHC != 0 || p.QH == 1) {
    TileRegs T;
    load_tile(mat + (int64_t)rb * kTileBytes, lane, T);
    float part[1][8];
    tile_dot_bf16<1>(T, xr, part);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = part[0][i];
    reduce_slabs_rt<LHC>(v, lane, L);
  } else {
    panels_dot_bf16<LHC>(mat, rb, p.QH, p.KpH, p.x, p.H, m, lane, L, v);
  }
  const int nv = LHC ? 1 : reduced_values(L);
#pragma unroll
  for (int q = 0; q < NV; ++q)
    if (wave == 1 && q < nv) up_lds[q][lane] = v[q];
  __syncthreads();
  if (wave == 0 && reduced_writer_rt(lane, L)) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      if (q < nv) {
        const int i = j * p.RH + reduced_row_v(lane, L, q);
        p.hp[(int64_t)item * p.I + i] = silu(v[q] * g) * (up_lds[q][lane] * g);
      }
    }
  }
}

}  // namespace nvfp4moe
