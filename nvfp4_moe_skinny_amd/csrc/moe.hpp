// moe.hpp - grouped skinny NVFP4 expert products and the routing-weighted combine.
//
// Work is addressed by expert slot: slot s < n_active is active expert
// active[s] with the (row, slot) pairs pairs[offsets[e] .. offsets[e+1]);
// slot `routed_slots` is the shared expert with every row. Nothing about the
// routing is read back to the host: blocks of slots past n_active exit.
//
// gate_up: one wave per (slot, gate tile j): it streams gate tile j and the
//   matching up tile j + I / rows_per_tile, keeps both in registers, and for
//   every row of the slot writes h = silu(u_gate) * u_up (FP32) to the
//   workspace.
// down:    one wave per (slot, down tile); four tiles per block. Each block
//   writes y = W_dn h (FP32) for its rows to the workspace, then bumps the
//   counter of its tile group; the last block to arrive for a group combines
//   out = sum_j w_j y_j (+ shared) (+ residual) in slot order and rounds once
//   to BF16. No floating-point atomics: the result does not depend on which
//   block arrives last.
#pragma once

#include "tile.hpp"

namespace nvfp4moe {

struct MoeParams {
  const uint16_t* x;
  const float* w;
  const int32_t* offsets;
  const int32_t* pairs;
  const int32_t* active;
  const int32_t* n_active;
  const uint8_t* gu;
  const uint8_t* dn;
  const uint8_t* sgu;
  const uint8_t* sdn;
  const uint16_t* residual;
  uint16_t* out;
  float* h;           // [P_tot][I]
  float* y;           // [P_tot][H]
  uint32_t* counters; // [dn_groups]
  int M, E, k, H, I;
  int routed_slots;
  int has_shared;
  int64_t gu_mat_bytes, dn_mat_bytes;
  const float* gu_g;  // [E] tensor scales inside the packed gate_up tensor
  const float* dn_g;
  const float* sgu_g;
  const float* sdn_g;
  int gu_tiles_per_half;   // I / rows_per_tile(H)
  int gu_blocks_per_slot;  // ceil(gu_tiles_per_half / 4)
  int dn_tiles;            // tiles_per_matrix(H, I)
  int dn_groups;           // ceil(dn_tiles / 4)
};

struct SlotInfo {
  int e;
  int row_begin;
  int rows;
  bool shared;
};

__device__ __forceinline__ bool slot_info(const MoeParams& p, int slot, SlotInfo& s) {
  if (slot < p.routed_slots) {
    if (slot >= *p.n_active) return false;
    s.e = p.active[slot];
    s.row_begin = p.offsets[s.e];
    s.rows = p.offsets[s.e + 1] - s.row_begin;
    s.shared = false;
  } else {
    s.e = 0;
    s.row_begin = 0;
    s.rows = p.M;
    s.shared = true;
  }
  return true;
}

// Pair index (row of h / y in the workspace) and activation row of row r of a slot.
__device__ __forceinline__ int slot_pair(const MoeParams& p, const SlotInfo& s, int r) {
  return s.shared ? p.M * p.k + r : p.pairs[s.row_begin + r];
}
__device__ __forceinline__ int pair_xrow(const MoeParams& p, int pair) {
  return pair >= p.M * p.k ? pair - p.M * p.k : pair / p.k;
}

// ---- gate_up + SiLU * up ---------------------------------------------------------------

template <int L, int R>
__device__ __forceinline__ void gate_up_rows(const MoeParams& p, const SlotInfo& s,
                                             const TileRegs& TG, const TileRegs& TU, int r0,
                                             int rows, int lane, int tile, float g) {
  const int col0 = 32 * (lane % L);
  int pr[R];
  uint4 xr[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r) : 0;
    load_x_bf16(p.x, p.H, pair_xrow(p, pr[r]), r < rows, col0, xr[r]);
  }
  float pg[R][8], pu[R][8];
  tile_dot_bf16<R>(TG, xr, pg);
  tile_dot_bf16<R>(TU, xr, pu);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    reduce_slabs<L>(pg[r], lane);
    reduce_slabs<L>(pu[r], lane);
  }
  if (!reduced_writer<L>(lane)) return;
  constexpr int rpt = 16384 / (L * 32);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= rows) break;
#pragma unroll
    for (int j = 0; j < reduced_count<L>(); ++j) {
      const int i = tile * rpt + tile_row<L>(reduced_slab<L>(lane) + j, lane);
      p.h[(int64_t)pr[r] * p.I + i] = silu(pg[r][j] * g) * (pu[r][j] * g);
    }
  }
}

template <int L>  // L = H / 32
__global__ void __launch_bounds__(256) moe_gate_up_kernel(MoeParams p) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < p.dn_groups; i += blockDim.x) p.counters[i] = 0u;
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.x / p.gu_blocks_per_slot;
  const int tile = (blockIdx.x % p.gu_blocks_per_slot) * 4 + (threadIdx.x >> 6);
  if (tile >= p.gu_tiles_per_half) return;
  SlotInfo s;
  if (!slot_info(p, slot, s)) return;
  const uint8_t* mat = s.shared ? p.sgu : p.gu + (int64_t)s.e * p.gu_mat_bytes;
  const float g = s.shared ? p.sgu_g[0] : p.gu_g[s.e];
  TileRegs TG, TU;
  load_tile(mat + (int64_t)tile * kTileBytes, lane, TG);
  load_tile(mat + (int64_t)(tile + p.gu_tiles_per_half) * kTileBytes, lane, TU);
  for (int r0 = 0; r0 < s.rows; r0 += 8) {
    const int rows = (s.rows - r0) < 8 ? (s.rows - r0) : 8;
    if (rows > 4)
      gate_up_rows<L, 8>(p, s, TG, TU, r0, rows, lane, tile, g);
    else if (rows > 2)
      gate_up_rows<L, 4>(p, s, TG, TU, r0, rows, lane, tile, g);
    else if (rows > 1)
      gate_up_rows<L, 2>(p, s, TG, TU, r0, rows, lane, tile, g);
    else
      gate_up_rows<L, 1>(p, s, TG, TU, r0, rows, lane, tile, g);
  }
}

// ---- down + combine ----------------------------------------------------------------------

template <int L, int R>
__device__ __forceinline__ void down_rows(const MoeParams& p, const SlotInfo& s,
                                          const TileRegs& T, int r0, int rows, int lane, int tile,
                                          float g) {
  const int col0 = 32 * (lane % L);
  int pr[R];
  float hr[R][32];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r) : 0;
    load_h_f32(p.h, p.I, pr[r], r < rows, col0, hr[r]);
  }
  float part[R][8];
  tile_dot_f32<R>(T, hr, part);
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs<L>(part[r], lane);
  if (!reduced_writer<L>(lane)) return;
  constexpr int rpt = 16384 / (L * 32);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= rows) break;
#pragma unroll
    for (int j = 0; j < reduced_count<L>(); ++j) {
      const int n = tile * rpt + tile_row<L>(reduced_slab<L>(lane) + j, lane);
      if (n < p.H) p.y[(int64_t)pr[r] * p.H + n] = part[r][j] * g;
    }
  }
}

template <int L>  // L = I / 32
__global__ void __launch_bounds__(256) moe_down_combine_kernel(MoeParams p) {
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.x / p.dn_groups;
  const int group = blockIdx.x % p.dn_groups;
  const int tile = group * 4 + (threadIdx.x >> 6);
  SlotInfo s;
  if (!slot_info(p, slot, s)) return;  // uniform over the block
  if (tile < p.dn_tiles) {
    const uint8_t* mat = s.shared ? p.sdn : p.dn + (int64_t)s.e * p.dn_mat_bytes;
    const float g = s.shared ? p.sdn_g[0] : p.dn_g[s.e];
    TileRegs T;
    load_tile(mat + (int64_t)tile * kTileBytes, lane, T);
    for (int r0 = 0; r0 < s.rows; r0 += 8) {
      const int rows = (s.rows - r0) < 8 ? (s.rows - r0) : 8;
      if (rows > 4)
        down_rows<L, 8>(p, s, T, r0, rows, lane, tile, g);
      else if (rows > 2)
        down_rows<L, 4>(p, s, T, r0, rows, lane, tile, g);
      else if (rows > 1)
        down_rows<L, 2>(p, s, T, r0, rows, lane, tile, g);
      else
        down_rows<L, 1>(p, s, T, r0, rows, lane, tile, g);
    }
  }
  // publish this block's y rows, then count arrivals for the tile group
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t participants = (uint32_t)(*p.n_active + p.has_shared);
    const uint32_t prev = __hip_atomic_fetch_add(&p.counters[group], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last = (prev + 1u == participants);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  constexpr int rpt = 16384 / (L * 32);
  const int n0 = group * 4 * rpt;
  const int n1 = (n0 + 4 * rpt) < p.H ? (n0 + 4 * rpt) : p.H;
  const int nrows = n1 - n0;
  for (int idx = threadIdx.x; idx < p.M * nrows; idx += blockDim.x) {
    const int m = idx / nrows;
    const int n = n0 + idx % nrows;
    float acc = 0.0f;
    for (int j = 0; j < p.k; ++j)
      acc += p.w[m * p.k + j] * p.y[(int64_t)(m * p.k + j) * p.H + n];
    if (p.has_shared) acc += p.y[(int64_t)(p.M * p.k + m) * p.H + n];
    if (p.residual) acc += bf16_to_f32(p.residual[(int64_t)m * p.H + n]);
    p.out[(int64_t)m * p.H + n] = f32_to_bf16_rne(acc);
  }
}

}  // namespace nvfp4moe
