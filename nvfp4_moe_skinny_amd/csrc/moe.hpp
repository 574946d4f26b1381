// moe.hpp - the routed NVFP4 MoE decode step in one launch:
//   gate_up -> SiLU * up -> down -> routing-weighted combine.
//
// Tiles: with rows_per_tile(K) = 16384 / K, the gate half of one expert's
// fused [2I][H] gate_up matrix and its [H][I] down matrix both hold
// P = H * I / 16384 tiles. Slot s < n_active is expert active[s] with the
// (row, slot) pairs pairs[offsets[e] .. offsets[e+1]); slot `routed_slots` is
// the shared expert over every row.
//
// One wavefront per block. Block w:
//   1. gate_up item w (slot w / P, tile j = w % P): streams gate tile j and up
//      tile P + j, multiplies them with the slot's rows in batches and writes
//      h = silu(u_gate) * u_up (FP32) for the tile's rows;
//   2. down item w - P (slot w / P - 1, tile w % P): streams that down tile,
//      waits until every gate_up item of its slot has published h, and
//      writes y = W_dn h (FP32) for the slot's rows; the last down item of an
//      output tile combines out = sum_j w_j y_j (+ shared) (+ residual) in
//      slot order and rounds once to BF16.
// The grid has (slots + 1) * P blocks. Nothing about the routing is read back
// to the host: items of slots past n_active return at once.
//
// Progress: a down item of slot s waits only for the gate_up items of slot s,
// which belong to blocks s * P .. s * P + P - 1, all below the waiter's index,
// and every block runs its gate_up item before its down item. Workgroups of a
// launch are dispatched to each XCD in increasing index order, so whatever a
// waiter depends on has been dispatched and publishes without waiting itself:
// every wait ends, whatever the residency. Each wait is also bounded: past
// spin_limit polls the block raises an error flag and carries on (the output
// is then invalid; the kernel still ends).
//
// Exchange: h and y travel as 64-bit words (FP32 value, 32-bit ready flag)
// written and read with single-copy-atomic, agent-scope (sc1) accesses, so a
// consumer polls the data itself and a producer never waits for its stores.
// The last consumer of a word clears it: the last down item of a slot (per
// slot counter) clears the slot's h rows, the combining block (last arrival
// on a per-output-tile counter) clears the y words it read. Every word and
// counter is therefore zero again when the launch ends (the workspace must be
// zero before the first launch). Device-scope atomics on one address
// serialise (~12 ns each on MI355X), so every counter sits on its own
// 128-byte line and there is no grid-wide counter.
#pragma once

#include "tile.hpp"

namespace nvfp4moe {

struct MoeParams {
  const uint16_t* x;
  const float* w;
  const int32_t* offsets;
  const int32_t* pairs;
  const int32_t* active;
  const int32_t* active_offsets;
  const int32_t* n_active;
  const uint8_t* gu;
  const uint8_t* dn;
  const uint8_t* sgu;
  const uint8_t* sdn;
  const uint16_t* residual;
  uint16_t* out;
  uint64_t* h;         // [P_tot][I] (value, ready) words
  uint64_t* y;         // [P_tot][H] (value, ready) words
  uint32_t* ctl;       // [2] error flag
  uint32_t* cnt_ds;    // per slot: down items done reading h  (stride kCounterStride)
  uint32_t* cnt_dn;    // per output tile: down items done     (stride kCounterStride)
  const float* gu_g;   // [E] tensor scales inside the packed gate_up tensor
  const float* dn_g;
  const float* sgu_g;
  const float* sdn_g;
  int64_t gu_mat_bytes, dn_mat_bytes;
  int M, E, k, H, I;
  int LH, LI;          // lanes per row: H / 32, I / 32
  int routed_slots, has_shared, slots;
  int P;               // tiles per gate half = tiles per down matrix = H * I / 16384
  int total_blocks;    // (slots + 1) * P
  uint32_t spin_limit;
};

constexpr int kCounterStride = 32;  // words: one 128-byte line per counter

// ---- agent-coherent accesses ---------------------------------------------------------

__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_coherent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(uint64_t* p, float v) {
  const uint64_t word = (1ull << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_word(uint64_t* p) {
  __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool word_ready(uint64_t w) { return (w >> 32) != 0; }
__device__ __forceinline__ float word_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Bounded back-off between polls; raises the error flag (once) past the limit.
struct Poller {
  uint32_t polls = 0;
  int nap = 1;
  __device__ __forceinline__ bool next(const MoeParams& p);
};

// Waits until this wave's outstanding memory operations (stores included) have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bool Poller::next(const MoeParams& p) {
  if (nap == 1) __builtin_amdgcn_s_sleep(1);
  else if (nap == 2) __builtin_amdgcn_s_sleep(2);
  else if (nap == 4) __builtin_amdgcn_s_sleep(4);
  else __builtin_amdgcn_s_sleep(8);
  nap = nap < 8 ? 2 * nap : 8;
  if (++polls > p.spin_limit) {
    store_coherent_u32(&p.ctl[2], 1u);
    return false;
  }
  return true;
}

// ---- slots ---------------------------------------------------------------------------

struct SlotInfo {
  int e;
  int row_begin;
  int rows;
  bool shared;
};

// One round trip: expert and row range of a slot from the per-slot arrays.
__device__ __forceinline__ bool slot_info(const MoeParams& p, int slot, SlotInfo& s) {
  if (slot < p.routed_slots) {
    const int e = p.active[slot];
    const int b = p.active_offsets[slot], en = p.active_offsets[slot + 1];
    if (e < 0) return false;
    s.e = e;
    s.row_begin = b;
    s.rows = en - b;
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

template <int LC, int R>
__device__ __forceinline__ void gate_up_batch(const MoeParams& p, const SlotInfo& s,
                                              const TileRegs& TG, const TileRegs& TU, int r0,
                                              int rows, int lane, int j, float g, int L) {
  const int col0 = 32 * (lane % L);
  int pr[R];
  uint4 xr[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r) : 0;
    load_x_bf16(p.x, p.H, pair_xrow(p, pr[r]), r < rows, col0, xr[r]);
  }
  float ug[R], uu[R];
  {
    float part[R][8];
    tile_dot_bf16<R>(TG, xr, part);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      reduce_slabs_rt<LC>(part[r], lane, L);
      ug[r] = part[r][0];
    }
  }
  {
    float part[R][8];
    tile_dot_bf16<R>(TU, xr, part);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      reduce_slabs_rt<LC>(part[r], lane, L);
      uu[r] = part[r][0];
    }
  }
  if (reduced_writer_rt(lane, L)) {
    const int i = j * (16384 / p.H) + reduced_row(lane, L);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rows) publish(&p.h[(int64_t)pr[r] * p.I + i], silu(ug[r] * g) * (uu[r] * g));
  }
}

template <int LC, int RMAX>
__device__ __forceinline__ void gate_up_compute(const MoeParams& p, int slot, const SlotInfo& s,
                                                int j, TileRegs& TG, TileRegs& TU, float g) {
  const int lane = threadIdx.x;
  const int L = LC ? LC : p.LH;
#pragma unroll 1
  for (int r0 = 0; r0 < s.rows; r0 += RMAX) {
    opaque_tile(TG);
    opaque_tile(TU);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      gate_up_batch<LC, (RMAX >= 8 ? 8 : 1)>(p, s, TG, TU, r0, rows, lane, j, g, L);
    else if (RMAX >= 4 && rows > 2)
      gate_up_batch<LC, (RMAX >= 4 ? 4 : 1)>(p, s, TG, TU, r0, rows, lane, j, g, L);
    else if (RMAX >= 2 && rows > 1)
      gate_up_batch<LC, (RMAX >= 2 ? 2 : 1)>(p, s, TG, TU, r0, rows, lane, j, g, L);
    else
      gate_up_batch<LC, 1>(p, s, TG, TU, r0, rows, lane, j, g, L);
  }
}

// ---- down + combine ---------------------------------------------------------------------------

template <int LC, int R>
__device__ __forceinline__ void down_batch(const MoeParams& p, const SlotInfo& s, const TileRegs& T,
                                           int r0, int rows, int lane, int tile, float g, int L,
                                           float* s_h) {
  // stage the batch's h rows in LDS, polling until every word is ready
  const int I = p.I;
  const int per_row = I / 64;  // words per lane per row
  Poller poll;
  for (int r = 0; r < R; ++r) {
    if (r >= rows) break;
    const uint64_t* src = p.h + (int64_t)slot_pair(p, s, r0 + r) * I;
    bool done = false;
    while (!done) {
      bool mine = true;
      for (int q = 0; q < per_row; ++q) {
        const int c = q * 64 + lane;
        const uint64_t wd = load_word(src + c);
        mine = mine && word_ready(wd);
        s_h[r * I + c] = word_value(wd);
      }
      done = __builtin_amdgcn_read_exec() == __ballot(mine);
      if (!done && !poll.next(p)) break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS writes have landed
  __builtin_amdgcn_wave_barrier();
  const int col0 = 32 * (lane % L);
  float hr[R][32];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float4* hp = reinterpret_cast<const float4*>(s_h + r * I + col0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = hp[q];
      hr[r][4 * q] = v.x;
      hr[r][4 * q + 1] = v.y;
      hr[r][4 * q + 2] = v.z;
      hr[r][4 * q + 3] = v.w;
    }
  }
  float part[R][8];
  tile_dot_f32<R>(T, hr, part);
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs_rt<LC>(part[r], lane, L);
  const int n = tile * (16384 / p.I) + reduced_row(lane, L);
  if (reduced_writer_rt(lane, L) && n < p.H) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rows) {
        const int pr = slot_pair(p, s, r0 + r);
        publish(&p.y[(int64_t)pr * p.H + n], part[r][0] * g);
      }
  }
  __builtin_amdgcn_wave_barrier();  // s_h is rewritten by the next batch
}

// y word of pair row `pr`, output n: polls until ready, then clears it (the
// combining block is its only reader).
__device__ __forceinline__ float take_y(const MoeParams& p, int pr, int n, Poller& poll) {
  uint64_t* a = &p.y[(int64_t)pr * p.H + n];
  uint64_t wd = load_word(a);
  while (!word_ready(wd)) {
    if (!poll.next(p)) break;
    wd = load_word(a);
  }
  clear_word(a);
  return word_value(wd);
}

// out rows of output tile t: sum over slots in j order, then shared, then residual.
__device__ __forceinline__ void combine_tile(const MoeParams& p, int tile) {
  const int rpt = 16384 / p.I;
  const int n0 = tile * rpt;
  const int n1 = (n0 + rpt) < p.H ? (n0 + rpt) : p.H;
  const int nrows = n1 - n0;
  Poller poll;
  for (int idx = threadIdx.x; idx < p.M * nrows; idx += 64) {
    const int m = idx / nrows;
    const int n = n0 + idx % nrows;
    float acc = 0.0f;
    for (int j = 0; j < p.k; ++j) acc += p.w[m * p.k + j] * take_y(p, m * p.k + j, n, poll);
    if (p.has_shared) acc += take_y(p, p.M * p.k + m, n, poll);
    if (p.residual) acc += bf16_to_f32(p.residual[(int64_t)m * p.H + n]);
    p.out[(int64_t)m * p.H + n] = f32_to_bf16_rne(acc);
  }
}

template <int LC, int RMAX>
__device__ __forceinline__ void down_compute(const MoeParams& p, int slot, const SlotInfo& s,
                                             int tile, TileRegs& T, float g, float* s_h) {
  const int lane = threadIdx.x;
  const int L = LC ? LC : p.LI;
#pragma unroll 1
  for (int r0 = 0; r0 < s.rows; r0 += RMAX) {
    opaque_tile(T);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      down_batch<LC, (RMAX >= 8 ? 8 : 1)>(p, s, T, r0, rows, lane, tile, g, L, s_h);
    else if (RMAX >= 4 && rows > 2)
      down_batch<LC, (RMAX >= 4 ? 4 : 1)>(p, s, T, r0, rows, lane, tile, g, L, s_h);
    else if (RMAX >= 2 && rows > 1)
      down_batch<LC, (RMAX >= 2 ? 2 : 1)>(p, s, T, r0, rows, lane, tile, g, L, s_h);
    else
      down_batch<LC, 1>(p, s, T, r0, rows, lane, tile, g, L, s_h);
  }
  // done reading the slot's h: the last reader clears the slot's h words
  int last_reader = 0;
  if (lane == 0)
    last_reader = add_coherent(&p.cnt_ds[slot * kCounterStride], 1u) + 1u == (uint32_t)p.P;
  if (__builtin_amdgcn_readfirstlane(last_reader)) {
    for (int r = 0; r < s.rows; ++r) {
      uint64_t* row = p.h + (int64_t)slot_pair(p, s, r) * p.I;
      for (int c = lane; c < p.I; c += 64) clear_word(row + c);
    }
    if (lane == 0) store_coherent_u32(&p.cnt_ds[slot * kCounterStride], 0u);
  }
  // y is published; the last down item of the output tile combines it
  int last = 0;
  if (lane == 0) {
    const uint32_t participants = (uint32_t)(*p.n_active + p.has_shared);
    last = add_coherent(&p.cnt_dn[tile * kCounterStride], 1u) + 1u == participants;
    if (last) store_coherent_u32(&p.cnt_dn[tile * kCounterStride], 0u);
  }
  if (__builtin_amdgcn_readfirstlane(last)) combine_tile(p, tile);
}

// ---- the kernel ----------------------------------------------------------------------------------

// One wave per block; dynamic LDS: RMAX rows of h (RMAX * I floats). The
// block reads both items' routing entries first, then issues all three
// tiles (gate, up, down) before any compute, so the only dependent memory
// round trip left on its path is the exchange of h.
template <int LHC, int LIC, int RMAX>
__global__ void __launch_bounds__(64) moe_decode_kernel(MoeParams p) {
  extern __shared__ float s_h[];
  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int gslot = w / p.P, dslot = w / p.P - 1, j = w % p.P;
  SlotInfo gs, ds;
  const bool has_gu = gslot < p.slots && slot_info(p, gslot, gs);
  const bool has_dn = dslot >= 0 && slot_info(p, dslot, ds);
  TileRegs TG, TU, TD;
  float ggu = 0.0f, gdn = 0.0f;
  if (has_gu) {
    const uint8_t* mat = gs.shared ? p.sgu : p.gu + (int64_t)gs.e * p.gu_mat_bytes;
    ggu = gs.shared ? p.sgu_g[0] : p.gu_g[gs.e];
    load_tile(mat + (int64_t)j * kTileBytes, lane, TG);
    load_tile(mat + (int64_t)(j + p.P) * kTileBytes, lane, TU);
  }
  if (has_dn) {
    const uint8_t* mat = ds.shared ? p.sdn : p.dn + (int64_t)ds.e * p.dn_mat_bytes;
    gdn = ds.shared ? p.sdn_g[0] : p.dn_g[ds.e];
    load_tile(mat + (int64_t)j * kTileBytes, lane, TD);
  }
  if (has_gu) gate_up_compute<LHC, RMAX>(p, gslot, gs, j, TG, TU, ggu);
  if (has_dn) down_compute<LIC, RMAX>(p, dslot, ds, j, TD, gdn, s_h);
}

}  // namespace nvfp4moe
