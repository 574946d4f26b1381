// fused.hpp - routing folded into gate_up for few rows (two launches from the
// logits to the output, with token_down_combine_kernel).
//
// One block per (item, gate tile j); items go row by row: row m's k slots,
// then (with a shared expert) its shared row. The launch's blocks are dealt to
// the XCDs in consecutive ranges, so in this order every XCD gets the same mix
// of routed and shared items; with the shared rows last, one XCD took nearly
// all of them (tiles its L2 already held) and ran idle for the last 5 of the
// launch's 17 us (40-layer stack 1207.6 -> 1194.5 us). Both waves of a routed
// item select the top k of row m themselves (the same per-row routine as
// moe_route_topk, so the same experts and weights bit for bit), then request
// row m of x; wave 0 streams gate tile j of expert ids[m][jj], wave 1 the up
// tile, as in staged_gate_split_kernel. The items
// of tile 0 store ids and w for the down launch. With few rows nearly every
// pair has its own expert, so a tile per pair costs almost no extra bytes, and
// no grouping is needed.
// SHARED (a shared expert present) is a template argument: without it the
// routing is not behind a per-item branch, which measured faster (M = 4:
// 15.44 -> 15.28 us per step; folding the shared rows into the slot-0 items
// instead of giving them their own: stack 1181 -> 1201 us).
#pragma once

#include "route.hpp"
#include "staged.hpp"

namespace nvfp4moe {

// At most six waves per SIMD: aiming for seven (71 VGPRs), the compiler
// issued eight of a tile's nine loads and the ninth only once the first had
// arrived and been decoded into its registers; at 73 VGPRs all nine go out
// together (M = 4: 15.28 -> 15.15 us per step; 40-layer stack unchanged;
// capped at four: stack 1181 -> 1234 us).
template <int LHC, bool SHARED>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(4, 6)))
fused_route_gate_kernel(MoeParams p, const float* __restrict__ logits,
                        const float* __restrict__ bias, int32_t* __restrict__ ids,
                        float* __restrict__ w) {
  constexpr int NV = LHC ? 1 : 8;  // reduced values a lane may hold
  __shared__ float up_lds[NV][64];
  __shared__ float lp[2][kRouteMaxE];
  __shared__ uint4 xls[2][LHC ? 4 * LHC : 1];  // each wave's row of x (LHC != 0)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = xcd_block((int)blockIdx.x, (int)gridDim.x);
  // H = 2048, I = 512: 512 / 8 gate row blocks, a constant without a shared
  // expert (with p.PG the division here measured 0.11 us more per M = 4 step;
  // with a shared expert the constant measured slower: 40-layer stack 1177.8
  // -> 1188.6 us)
  const int PG = (LHC == 64 && !SHARED) ? 64 : p.PG;
  const int item = b / PG, j = b % PG;
  const int npairs = p.M * p.k;
  const int nq = SHARED ? p.k + 1 : p.k;  // row m's items: its k slots, then its shared row
  const int m = item / nq, q = item - m * nq;
  const bool sh = SHARED && q == p.k;
  const int hrow = sh ? npairs + m : m * p.k + q;  // the pair's h row
  const int L = LHC ? LHC : p.LH;
  uint4 xr[1][4];
  // Row m of x. At H = 2048 (LHC = 64) the wave requests the 4 KB row in
  // coalesced 1 KB pieces once its routing is done and reads its lane's 64
  // bytes back from its LDS row when the tile's loads are out (against direct
  // loads, before the routing with a shared expert: 40-layer stack 1147.5 ->
  // 1138.3 us; without one, after it: M = 4 unchanged). The generic instance
  // loads the lane's columns directly: before the routing with a shared
  // expert, after its wait without one (with direct loads at H = 2048: M = 4
  // 15.025 -> 14.967 us late; the 40-layer stack 1179.6 -> 1190.8 us late).
  if constexpr (SHARED && LHC == 0) load_x_bf16(p.x, p.H, m, 32 * (lane % L), xr[0]);
  int e = 0;
  if (!sh) {
    int my_id;
    float my_w;
    const int jj = q;
    // the items of tile 0 store ids and w (all k rounds, softmax); the others
    // need only the first jj + 1 experts
    // with a shared expert (a launch of more blocks than fit at once), waves
    // with more selection rounds ahead issue first while routing (40-layer
    // stack 1174.9 -> 1164.0 us; without one, M = 4 measured 14.95 -> 15.53)
    if constexpr (SHARED) {
      if (j == 0 || jj >= 6) __builtin_amdgcn_s_setprio(3);
      else if (jj >= 3) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(1);
    }
    route_row_core(logits, bias, p.E, p.k, m, lane, lp[wave], my_id, my_w,
                   j == 0 ? kRouteMaxK : jj + 1, j == 0);
    if constexpr (SHARED) __builtin_amdgcn_s_setprio(0);
    e = __builtin_amdgcn_readlane(my_id, jj);
    if (j == 0 && wave == 0 && lane == jj) {
      ids[hrow] = my_id;
      w[hrow] = my_w;
    }
  }
  uint4 xv[LHC ? LHC / 16 : 1];
  if constexpr (LHC != 0)
    load_coalesced(reinterpret_cast<const uint4*>(p.x + (int64_t)m * p.H), lane, xv);
  else if constexpr (!SHARED)
    load_x_bf16(p.x, p.H, m, 32 * (lane % L), xr[0]);
  const uint8_t* mat = sh ? p.sgu : p.gu + (int64_t)e * p.gu_mat_bytes;
  const float g = sh ? p.sgu_g[0] : p.gu_g[e];
  const int rb = wave == 0 ? j : j + PG;  // gate row block j, or the matching up one
  float v[8];
  if (LHC != 0 || p.QH == 1) {
    TileRegs T;
    // without a shared expert the tile's scale word goes first, so that a
    // slab's scaled sum does not wait for the last load (M = 4: 14.705 ->
    // 14.688 us; measured slower before x came in coalesced pieces, 15.12 ->
    // 15.22 us)
    if constexpr (LHC != 0 && !SHARED)
      load_tile_scales_first(mat + (int64_t)rb * kTileBytes, lane, T);
    else
      load_tile(mat + (int64_t)rb * kTileBytes, lane, T);
    if constexpr (LHC != 0) restage_row(xls[wave], lane, lane % LHC, xv, xr[0]);
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
  for (int qv = 0; qv < NV; ++qv)
    if (wave == 1 && qv < nv) up_lds[qv][lane] = v[qv];
  __syncthreads();
  if (wave == 0 && reduced_writer_rt(lane, L)) {
#pragma unroll
    for (int qv = 0; qv < NV; ++qv) {
      if (qv < nv) {
        const int i = j * p.RH + reduced_row_v(lane, L, qv);
        p.hp[(int64_t)hrow * p.I + i] = silu(v[qv] * g) * (up_lds[qv][lane] * g);
      }
    }
  }
}

}  // namespace nvfp4moe
