// moe.hpp - the routed NVFP4 MoE decode step in one launch:
//   gate_up -> SiLU * up -> down -> routing-weighted combine.
//
// Work items (one 128-thread block each, two waves):
//   gate_up item (slot, j): wave 0 streams gate tile j, wave 1 up tile j
//     (j + I / rows_per_tile(H) in the fused [2I][H] matrix); both keep their
//     tile in registers and pass over the slot's rows in batches; wave 1 hands
//     its reduced up values to wave 0 through LDS, wave 0 writes
//     h = silu(u_gate) * u_up (FP32) for the tile's rows.
//   down item (slot, group): waits until every gate_up item of its slot has
//     published h, then each wave streams one down tile and writes y = W_dn h
//     (FP32) for the slot's rows; the last down item to finish an output group
//     combines out = sum_j w_j y_j (+ shared) (+ residual) in slot order and
//     rounds once to BF16.
// Slot s < n_active is expert active[s] with pairs pairs[offsets[e] ..
// offsets[e+1]); slot `routed_slots` is the shared expert over every row.
// Nothing about the routing is read back to the host.
//
// Ordering and progress: each block takes a ticket from a counter when it
// starts; tickets below gu_items are gate_up items, the rest down items. A
// block only ever waits on items with smaller tickets, which have started
// and never wait themselves, so the grid cannot deadlock whatever order the
// hardware dispatches blocks in. Every wait is bounded: past spin_limit polls
// the block raises an error flag and carries on (results are then wrong, the
// kernel still ends).
//
// Coherence across the XCDs' L2 caches: h, y and the counters are written and
// read with agent-scope (sc1) accesses; a writer waits for its stores to
// complete (s_waitcnt vmcnt(0)) before bumping a counter. No cache flush is
// needed. The last block to finish resets every counter, so the workspace's
// control words are zero again when the launch ends (they must be zero before
// the first launch).
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
  float* h;            // [P_tot][I]
  float* y;            // [P_tot][H]
  uint32_t* ctl;       // [0] ticket, [1] finished blocks, [2] error flag
  uint32_t* cnt_gu;    // [slots] gate_up items done per slot
  uint32_t* cnt_dn;    // [dn_groups] down items done per output group
  const float* gu_g;   // [E] tensor scales inside the packed gate_up tensor
  const float* dn_g;
  const float* sgu_g;
  const float* sdn_g;
  int64_t gu_mat_bytes, dn_mat_bytes;
  int M, E, k, H, I;
  int LH, LI;          // lanes per row: H / 32, I / 32
  int routed_slots, has_shared, slots;
  int gu_pairs;        // gate tiles per slot = I / rows_per_tile(H)
  int dn_tiles;        // tiles_per_matrix(H, I)
  int dn_groups;       // ceil(dn_tiles / 2)
  int gu_items, dn_items, total_blocks;
  uint32_t spin_limit;
};

// ---- agent-coherent accesses ---------------------------------------------------------

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_coherent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's outstanding memory operations (stores included) have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- slots ---------------------------------------------------------------------------

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

// Workspace row (pair index) and activation row of row r of a slot.
__device__ __forceinline__ int slot_pair(const MoeParams& p, const SlotInfo& s, int r) {
  return s.shared ? p.M * p.k + r : p.pairs[s.row_begin + r];
}
__device__ __forceinline__ int pair_xrow(const MoeParams& p, int pair) {
  return pair >= p.M * p.k ? pair - p.M * p.k : pair / p.k;
}

// ---- segmented reduction with a runtime row width (L >= 8) ----------------------------

// After: v[0] of lane l holds the full sum for slab ((l & (L-1)) >> (log2 L - 3)),
// identical in the L/8 lanes of its group.
template <int LC>
__device__ __forceinline__ void reduce_slabs_rt(float (&v)[8], int lane, int Lrt) {
  if constexpr (LC != 0) {
    reduce_slabs<LC>(v, lane);
  } else {
    int count = 8;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int d = Lrt >> (t + 1);
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
    for (int d = Lrt / 16; d >= 1; d >>= 1) v[0] += xor_shuffle(v[0], d);
  }
}

__device__ __forceinline__ int log2i(int v) { return 31 - __builtin_clz(v); }

// (tile row, writer?) of the reduced value held by `lane` for row width L >= 8.
__device__ __forceinline__ int reduced_row(int lane, int L) {
  const int slab = ((lane & (L - 1)) >> (log2i(L) - 3)) & 7;
  return slab * (64 / L) + lane / L;
}
__device__ __forceinline__ bool reduced_writer_rt(int lane, int L) {
  return (lane & (L / 8 - 1)) == 0;
}

// ---- gate_up + SiLU * up ------------------------------------------------------------------

template <int LC, int R, int RMAX>
__device__ __forceinline__ void gate_up_batch(const MoeParams& p, const SlotInfo& s,
                                              const TileRegs& T, int r0, int rows, int lane,
                                              int wave, int pair_tile, float g, int L,
                                              float (*s_up)[64]) {
  const int col0 = 32 * (lane % L);
  int pr[R];
  uint4 xr[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r) : 0;
    load_x_bf16(p.x, p.H, pair_xrow(p, pr[r]), r < rows, col0, xr[r]);
  }
  float part[R][8];
  tile_dot_bf16<R>(T, xr, part);
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs_rt<LC>(part[r], lane, L);
  const int row = reduced_row(lane, L);
  const bool writer = reduced_writer_rt(lane, L);
  if (wave == 1 && writer) {
#pragma unroll
    for (int r = 0; r < R; ++r) s_up[r][row] = part[r][0] * g;
  }
  __syncthreads();
  if (wave == 0 && writer) {
    const int rpt = 16384 / p.H;
    const int i = pair_tile * rpt + row;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rows) store_coherent(&p.h[(int64_t)pr[r] * p.I + i], silu(part[r][0] * g) * s_up[r][row]);
  }
  __syncthreads();
}

template <int LC, int RMAX>
__device__ __forceinline__ void gate_up_item(const MoeParams& p, int item, float (*s_up)[64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = item / p.gu_pairs;
  const int j = item % p.gu_pairs;
  SlotInfo s;
  if (!slot_info(p, slot, s)) return;  // uniform over the block
  const int L = LC ? LC : p.LH;
  const uint8_t* mat = s.shared ? p.sgu : p.gu + (int64_t)s.e * p.gu_mat_bytes;
  const float g = s.shared ? p.sgu_g[0] : p.gu_g[s.e];
  TileRegs T;
  load_tile(mat + (int64_t)(j + wave * p.gu_pairs) * kTileBytes, lane, T);
#pragma unroll 1
  for (int r0 = 0; r0 < s.rows; r0 += RMAX) {
    opaque_tile(T);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      gate_up_batch<LC, (RMAX >= 8 ? 8 : 1), RMAX>(p, s, T, r0, rows, lane, wave, j, g, L, s_up);
    else if (RMAX >= 4 && rows > 2)
      gate_up_batch<LC, (RMAX >= 4 ? 4 : 1), RMAX>(p, s, T, r0, rows, lane, wave, j, g, L, s_up);
    else if (RMAX >= 2 && rows > 1)
      gate_up_batch<LC, (RMAX >= 2 ? 2 : 1), RMAX>(p, s, T, r0, rows, lane, wave, j, g, L, s_up);
    else
      gate_up_batch<LC, 1, RMAX>(p, s, T, r0, rows, lane, wave, j, g, L, s_up);
  }
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) add_coherent(&p.cnt_gu[slot], 1u);
}

// ---- down + combine ---------------------------------------------------------------------------

template <int LC, int R>
__device__ __forceinline__ void down_batch(const MoeParams& p, const SlotInfo& s, const TileRegs& T,
                                           int r0, int rows, int lane, int tile, float g, int L) {
  const int col0 = 32 * (lane % L);
  int pr[R];
  float hr[R][32];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r) : 0;
    const float* hp = p.h + (int64_t)pr[r] * p.I + col0;
#pragma unroll
    for (int c = 0; c < 32; ++c) hr[r][c] = r < rows ? load_coherent(hp + c) : 0.0f;
  }
  float part[R][8];
  tile_dot_f32<R>(T, hr, part);
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs_rt<LC>(part[r], lane, L);
  if (!reduced_writer_rt(lane, L)) return;
  const int n = tile * (16384 / p.I) + reduced_row(lane, L);
  if (n >= p.H) return;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < rows) store_coherent(&p.y[(int64_t)pr[r] * p.H + n], part[r][0] * g);
}

__device__ __forceinline__ void combine_group(const MoeParams& p, int group) {
  const int rpt = 16384 / p.I;
  const int n0 = group * 2 * rpt;
  const int n1 = (n0 + 2 * rpt) < p.H ? (n0 + 2 * rpt) : p.H;
  const int nrows = n1 - n0;
  for (int idx = threadIdx.x; idx < p.M * nrows; idx += blockDim.x) {
    const int m = idx / nrows;
    const int n = n0 + idx % nrows;
    float acc = 0.0f;
    for (int j = 0; j < p.k; ++j)
      acc += p.w[m * p.k + j] * load_coherent(&p.y[(int64_t)(m * p.k + j) * p.H + n]);
    if (p.has_shared) acc += load_coherent(&p.y[(int64_t)(p.M * p.k + m) * p.H + n]);
    if (p.residual) acc += bf16_to_f32(p.residual[(int64_t)m * p.H + n]);
    p.out[(int64_t)m * p.H + n] = f32_to_bf16_rne(acc);
  }
}

template <int LC, int RMAX>
__device__ __forceinline__ void down_item(const MoeParams& p, int item, int* s_flag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = item / p.dn_groups;
  const int group = item % p.dn_groups;
  SlotInfo s;
  if (!slot_info(p, slot, s)) return;  // uniform over the block
  const int L = LC ? LC : p.LI;
  const int tile = 2 * group + wave;
  const uint8_t* mat = s.shared ? p.sdn : p.dn + (int64_t)s.e * p.dn_mat_bytes;
  const float g = s.shared ? p.sdn_g[0] : p.dn_g[s.e];
  // the tile does not depend on h: start streaming it before waiting
  TileRegs T;
  if (tile < p.dn_tiles) load_tile(mat + (int64_t)tile * kTileBytes, lane, T);
  if (threadIdx.x == 0) {
    uint32_t polls = 0;
    while (load_coherent_u32(&p.cnt_gu[slot]) < (uint32_t)p.gu_pairs) {
      __builtin_amdgcn_s_sleep(1);
      if (++polls > p.spin_limit) {
        store_coherent_u32(&p.ctl[2], 1u);
        break;
      }
    }
  }
  __syncthreads();
  if (tile < p.dn_tiles) {
#pragma unroll 1
    for (int r0 = 0; r0 < s.rows; r0 += RMAX) {
      opaque_tile(T);
      const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
      if (RMAX >= 8 && rows > 4)
        down_batch<LC, (RMAX >= 8 ? 8 : 1)>(p, s, T, r0, rows, lane, tile, g, L);
      else if (RMAX >= 4 && rows > 2)
        down_batch<LC, (RMAX >= 4 ? 4 : 1)>(p, s, T, r0, rows, lane, tile, g, L);
      else if (RMAX >= 2 && rows > 1)
        down_batch<LC, (RMAX >= 2 ? 2 : 1)>(p, s, T, r0, rows, lane, tile, g, L);
      else
        down_batch<LC, 1>(p, s, T, r0, rows, lane, tile, g, L);
    }
  }
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t participants = (uint32_t)(*p.n_active + p.has_shared);
    *s_flag = (add_coherent(&p.cnt_dn[group], 1u) + 1u == participants);
  }
  __syncthreads();
  if (*s_flag) combine_group(p, group);
}

// ---- the kernel ----------------------------------------------------------------------------------

template <int LHC, int LIC, int RMAX>
__global__ void __launch_bounds__(128) moe_decode_kernel(MoeParams p) {
  __shared__ uint32_t s_ticket;
  __shared__ int s_flag;
  __shared__ float s_up[RMAX][64];
  if (threadIdx.x == 0) s_ticket = add_coherent(&p.ctl[0], 1u);
  __syncthreads();
  const int t = (int)s_ticket;
  if (t < p.gu_items)
    gate_up_item<LHC, RMAX>(p, t, s_up);
  else if (t < p.gu_items + p.dn_items)
    down_item<LIC, RMAX>(p, t - p.gu_items, &s_flag);
  // the last block to finish leaves every control word at zero
  __syncthreads();
  if (threadIdx.x == 0) {
    if (add_coherent(&p.ctl[1], 1u) + 1u == (uint32_t)p.total_blocks) {
      for (int i = 0; i < p.slots; ++i) store_coherent_u32(&p.cnt_gu[i], 0u);
      for (int i = 0; i < p.dn_groups; ++i) store_coherent_u32(&p.cnt_dn[i], 0u);
      store_coherent_u32(&p.ctl[0], 0u);
      store_coherent_u32(&p.ctl[1], 0u);
    }
  }
}

}  // namespace nvfp4moe
