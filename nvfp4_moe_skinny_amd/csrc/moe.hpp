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
  const int32_t* ids;
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
  int pair_regs;       // ceil(M * k / 64) <= 2: pairs[] is held in registers; else 0
  // three-launch schedule (staged.hpp)
  float* hp;           // [P_tot][I] h words (FP32, or hi / lo BF16 for MFMA slots)
  float* yp;           // [P_tot][H] expert outputs (FP32)
  int dense_min_rows;  // slots with at least this many rows use MFMA
  // optional dense projection of x, computed by the first proj_blocks blocks
  // of the down launch (token_down_combine_kernel): py [M][pn] = x W_p^T
  const uint8_t* pw;
  uint16_t* py;
  int64_t pn;
  int proj_blocks;     // a multiple of 8 (0: none), so the XCD order of the rest holds
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

// pairs[] in registers (entry q * 64 + l in v[q] of lane l) when M * k <= 128:
// loaded in the same round trip as the slot's routing entries, so the first
// activation rows can be requested before the weight tiles.
struct PairCache {
  int v[2];
};

__device__ __forceinline__ void load_pair_cache(const MoeParams& p, int lane, PairCache& c) {
  const int n = p.M * p.k;
#pragma unroll
  for (int q = 0; q < 2; ++q)
    c.v[q] = (q < p.pair_regs && q * 64 + lane < n) ? p.pairs[q * 64 + lane] : 0;
}

// Reads another lane's register: call with every lane of the wave active (in
// a branch, the source lane's value may not have been copied where it is read).
__device__ __forceinline__ int cached_pair(const PairCache& c, int idx) {
  idx = __builtin_amdgcn_readfirstlane(idx);
  const int l = idx & 63;
  return idx < 64 ? __builtin_amdgcn_readlane(c.v[0], l) : __builtin_amdgcn_readlane(c.v[1], l);
}

// Workspace row (pair index) and activation row of row r of a slot.
__device__ __forceinline__ int slot_pair(const MoeParams& p, const SlotInfo& s, int r,
                                         const PairCache& c) {
  if (s.shared) return p.M * p.k + r;
  return p.pair_regs ? cached_pair(c, s.row_begin + r) : p.pairs[s.row_begin + r];
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
      const int half = count >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < half) v[j] = halve(v[j], v[j + half], d, lane);
      }
      count = half;
    }
    for (int d = Lrt / 16; d >= 1; d >>= 1) v[0] = fold(v[0], d, lane);
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

// h for R rows whose activations xr / pair ids pr are loaded: gate tile, up
// tile, h stores, then `after()` (the caller's hook, e.g. the next tile request).
template <int LC, int R, class After>
__device__ __forceinline__ void gate_up_rows(const MoeParams& p, const TileRegs& TG,
                                             const TileRegs& TU, const uint4 (&xr)[R][4],
                                             const int (&pr)[R], int rows, int lane, int j,
                                             float g, int L, After after) {
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
  after();
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Pair ids and activation rows r0 .. r0 + R - 1 of a slot (rows past `rows` are zero).
template <int R>
__device__ __forceinline__ void load_rows(const MoeParams& p, const SlotInfo& s,
                                          const PairCache& c, int r0, int rows, int col0,
                                          int (&pr)[R], uint4 (&xr)[R][4]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r, c) : 0;
    load_x_bf16(p.x, p.H, pair_xrow(p, pr[r]), r < rows, col0, xr[r]);
  }
}

template <int LC, int R>
__device__ __forceinline__ void gate_up_batch(const MoeParams& p, const SlotInfo& s,
                                              const PairCache& c, const TileRegs& TG,
                                              const TileRegs& TU, int r0, int rows, int lane,
                                              int j, float g, int L) {
  int pr[R];
  uint4 xr[R][4];
  load_rows<R>(p, s, c, r0, rows, 32 * (lane % L), pr, xr);
  gate_up_rows<LC, R>(p, TG, TU, xr, pr, rows, lane, j, g, L, NoHook{});
}

// Row batches from r0 on; the tile registers are made opaque per batch.
template <int LC, int RMAX>
__device__ __forceinline__ void gate_up_compute(const MoeParams& p, const SlotInfo& s,
                                                const PairCache& c, int r_begin, int j,
                                                TileRegs& TG, TileRegs& TU, float g) {
  const int lane = threadIdx.x;
  const int L = LC ? LC : p.LH;
#pragma unroll 1
  for (int r0 = r_begin; r0 < s.rows; r0 += RMAX) {
    opaque_tile(TG);
    opaque_tile(TU);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      gate_up_batch<LC, (RMAX >= 8 ? 8 : 1)>(p, s, c, TG, TU, r0, rows, lane, j, g, L);
    else if (RMAX >= 4 && rows > 2)
      gate_up_batch<LC, (RMAX >= 4 ? 4 : 1)>(p, s, c, TG, TU, r0, rows, lane, j, g, L);
    else if (RMAX >= 2 && rows > 1)
      gate_up_batch<LC, (RMAX >= 2 ? 2 : 1)>(p, s, c, TG, TU, r0, rows, lane, j, g, L);
    else
      gate_up_batch<LC, 1>(p, s, c, TG, TU, r0, rows, lane, j, g, L);
  }
}

// ---- down + combine ---------------------------------------------------------------------------

template <int LC, int R>
__device__ __forceinline__ void down_batch(const MoeParams& p, const SlotInfo& s,
                                           const PairCache& c, const TileRegs& T, int r0,
                                           int rows, int lane, int tile, float g, int L,
                                           float* s_h) {
  // Stage the batch's h rows in LDS: every row's words are loaded in one
  // round trip. While some are not ready the block polls only one word per
  // gate_up item and row (an item stores its h segment of a row with one
  // instruction), then loads the rows again: waiting blocks would otherwise
  // re-read whole rows and crowd the memory system the weights stream through.
  const int I = p.I;
  const int seg = 16384 / p.H;  // h words per gate_up item
  const int per_row = I / 64;  // words per lane per row
  int pr[R];
  const uint64_t* src[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = slot_pair(p, s, r0 + (r < rows ? r : 0), c);
    src[r] = p.h + (int64_t)pr[r] * I;
  }
  Poller poll;
  bool waiting = true;
  while (waiting) {
    bool mine = true;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows) {
        for (int q = 0; q < per_row; ++q) {
          const int c = q * 64 + lane;
          const uint64_t wd = load_word(src[r] + c);
          mine = mine && word_ready(wd);
          s_h[r * I + c] = word_value(wd);
        }
      }
    }
    if (__ballot(!mine) == 0) break;
    for (;;) {  // sentinel words until every item's has arrived
      if (!poll.next(p)) {
        waiting = false;
        break;
      }
      bool seen = true;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r < rows)
          for (int it = lane; it < p.P; it += 64)
            seen = seen && word_ready(load_word(src[r] + it * seg));
      if (__ballot(!seen) == 0) break;
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
      if (r < rows) publish(&p.y[(int64_t)pr[r] * p.H + n], part[r][0] * g);
  }
  __builtin_amdgcn_wave_barrier();  // s_h is rewritten by the next batch
}

// out rows of output tile t: sum over slots in j order, then shared, then
// residual. A lane takes up to kCombineBatch outputs at a time and loads all
// their y words, routing weights and residual values in one round trip; only
// words not yet ready are polled again. The combining block is the y words'
// only reader, so it clears them.
constexpr int kMaxTerms = 9;  // k <= 8 routed slots + the shared expert
constexpr int kCombineBatch = 4;

__device__ __forceinline__ void combine_tile(const MoeParams& p, int tile) {
  const int rpt = 16384 / p.I;
  const int n0 = tile * rpt;
  const int n1 = (n0 + rpt) < p.H ? (n0 + rpt) : p.H;
  const int nrows = n1 - n0;
  const int terms = p.k + p.has_shared;
  const int total = p.M * nrows;
  Poller poll;
  for (int base = 0; base < total; base += 64 * kCombineBatch) {
    uint64_t wd[kCombineBatch][kMaxTerms];
    float wt[kCombineBatch][kMaxTerms];
    float res[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int idx = base + b * 64 + (int)threadIdx.x;
      const int m = idx / nrows, n = n0 + idx % nrows;
      res[b] = (idx < total && p.residual) ? bf16_to_f32(p.residual[(int64_t)m * p.H + n]) : 0.0f;
#pragma unroll
      for (int t = 0; t < kMaxTerms; ++t) {
        wd[b][t] = 0;
        wt[b][t] = 0.0f;
        if (idx < total && t < terms) {
          const int pr = t < p.k ? m * p.k + t : p.M * p.k + m;
          wd[b][t] = load_word(&p.y[(int64_t)pr * p.H + n]);
          wt[b][t] = t < p.k ? p.w[m * p.k + t] : 1.0f;
        }
      }
    }
    // every load has returned before any store is issued: loads and stores
    // share one counter, so a wait for a load issued after a store would
    // also wait for that store's round trip
    float acc[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int idx = base + b * 64 + (int)threadIdx.x;
      const int m = idx / nrows, n = n0 + idx % nrows;
      acc[b] = 0.0f;
#pragma unroll
      for (int t = 0; t < kMaxTerms; ++t) {
        if (idx < total && t < terms) {
          const int pr = t < p.k ? m * p.k + t : p.M * p.k + m;
          const uint64_t* a = &p.y[(int64_t)pr * p.H + n];
          while (!word_ready(wd[b][t])) {
            if (!poll.next(p)) break;
            wd[b][t] = load_word(a);
          }
          acc[b] += wt[b][t] * word_value(wd[b][t]);  // routed slots in j order, then shared
        }
      }
      if (p.residual) acc[b] += res[b];
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int idx = base + b * 64 + (int)threadIdx.x;
      if (idx >= total) continue;
      const int m = idx / nrows, n = n0 + idx % nrows;
#pragma unroll
      for (int t = 0; t < kMaxTerms; ++t) {
        if (t < terms) {
          const int pr = t < p.k ? m * p.k + t : p.M * p.k + m;
          clear_word(&p.y[(int64_t)pr * p.H + n]);
        }
      }
      p.out[(int64_t)m * p.H + n] = f32_to_bf16_rne(acc[b]);
    }
  }
}

template <int LC, int RMAX>
__device__ __forceinline__ void down_compute(const MoeParams& p, int slot, const SlotInfo& s,
                                             const PairCache& c, int tile, TileRegs& T, float g,
                                             float* s_h) {
  const int lane = threadIdx.x;
  const int L = LC ? LC : p.LI;
#pragma unroll 1
  for (int r0 = 0; r0 < s.rows; r0 += RMAX) {
    opaque_tile(T);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      down_batch<LC, (RMAX >= 8 ? 8 : 1)>(p, s, c, T, r0, rows, lane, tile, g, L, s_h);
    else if (RMAX >= 4 && rows > 2)
      down_batch<LC, (RMAX >= 4 ? 4 : 1)>(p, s, c, T, r0, rows, lane, tile, g, L, s_h);
    else if (RMAX >= 2 && rows > 1)
      down_batch<LC, (RMAX >= 2 ? 2 : 1)>(p, s, c, T, r0, rows, lane, tile, g, L, s_h);
    else
      down_batch<LC, 1>(p, s, c, T, r0, rows, lane, tile, g, L, s_h);
  }
  // y is published and the slot's h has been read: count both at once. The
  // last down item of the output tile combines it; the last reader of the
  // slot's h clears those words.
  int last = 0, last_reader = 0;
  if (lane == 0) {
    const uint32_t participants = (uint32_t)(*p.n_active + p.has_shared);
    const uint32_t t_prev = add_coherent(&p.cnt_dn[tile * kCounterStride], 1u);
    const uint32_t r_prev = add_coherent(&p.cnt_ds[slot * kCounterStride], 1u);
    last = t_prev + 1u == participants;
    last_reader = r_prev + 1u == (uint32_t)p.P;
    if (last) store_coherent_u32(&p.cnt_dn[tile * kCounterStride], 0u);
    if (last_reader) store_coherent_u32(&p.cnt_ds[slot * kCounterStride], 0u);
  }
  if (__builtin_amdgcn_readfirstlane(last)) combine_tile(p, tile);
  if (__builtin_amdgcn_readfirstlane(last_reader)) {
    for (int r = 0; r < s.rows; ++r) {
      uint64_t* row = p.h + (int64_t)slot_pair(p, s, r, c) * p.I;
      for (int c = lane; c < p.I; c += 64) clear_word(row + c);
    }
  }
}

// ---- the kernel ----------------------------------------------------------------------------------

// Gate and up tiles in one interleaved request stream, scales first, so that
// slab i of both tiles has arrived once the loads issued before it have.
__device__ __forceinline__ void load_tile_pair(const uint8_t* a, const uint8_t* b, int lane,
                                               TileRegs& ta, TileRegs& tb) {
  ta.scales = load_stream(reinterpret_cast<const uint4*>(a + kTileCodeBytes) + lane);
  tb.scales = load_stream(reinterpret_cast<const uint4*>(b + kTileCodeBytes) + lane);
  const uint4* ca = reinterpret_cast<const uint4*>(a);
  const uint4* cb = reinterpret_cast<const uint4*>(b);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ta.codes[i] = load_stream(ca + i * 64 + lane);
    tb.codes[i] = load_stream(cb + i * 64 + lane);
  }
}

struct IssueTile {
  const uint8_t* tile;
  TileRegs* t;
  __device__ __forceinline__ void operator()() const {
    if (tile) {
      __builtin_amdgcn_sched_barrier(0);
      load_tile(tile, threadIdx.x, *t);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// One wave per block; dynamic LDS: RMAX rows of h (RMAX * I floats).
//   1. one round trip: both items' routing entries and (M * k <= 128) pairs[];
//   2. the first gate_up batch's activation rows, then the gate and up tiles;
//   3. slab i of each tile is multiplied as soon as it has arrived; h of the
//      first batch is stored; further row batches;
//   4. only then is the down tile requested (once the memory queues are full
//      a request stalls its wave until there is room, which must not delay the
//      h that other blocks wait for), and the down item runs.
// Blocks with at most two rows per batch take this path; wider batches load
// their rows after the tiles.
template <int LHC, int LIC, int RMAX>
__global__ void __launch_bounds__(64) moe_decode_kernel(MoeParams p) {
  extern __shared__ float s_h[];
  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int gslot = w / p.P, dslot = w / p.P - 1, j = w % p.P;
  PairCache pc;
  load_pair_cache(p, lane, pc);
  SlotInfo gs, ds;
  const bool has_gu = gslot < p.slots && slot_info(p, gslot, gs);
  const bool has_dn = dslot >= 0 && slot_info(p, dslot, ds);
  TileRegs TG, TU, TD;
  float gdn = 0.0f;
  const uint8_t* dtile = nullptr;
  if (has_dn) {
    const uint8_t* mat = ds.shared ? p.sdn : p.dn + (int64_t)ds.e * p.dn_mat_bytes;
    gdn = ds.shared ? p.sdn_g[0] : p.dn_g[ds.e];
    dtile = mat + (int64_t)j * kTileBytes;
  }
  if (has_gu) {
    const uint8_t* mat = gs.shared ? p.sgu : p.gu + (int64_t)gs.e * p.gu_mat_bytes;
    const float ggu = gs.shared ? p.sgu_g[0] : p.gu_g[gs.e];
    const uint8_t* tg = mat + (int64_t)j * kTileBytes;
    const uint8_t* tu = mat + (int64_t)(j + p.P) * kTileBytes;
    if constexpr (RMAX <= 2) {
      const int L = LHC ? LHC : p.LH;
      const int rows0 = gs.rows < RMAX ? gs.rows : RMAX;
      int pr[RMAX];
      uint4 xr[RMAX][4];
      load_rows<RMAX>(p, gs, pc, 0, rows0, 32 * (lane % L), pr, xr);
      __builtin_amdgcn_sched_barrier(0);
      load_tile_pair(tg, tu, lane, TG, TU);
      __builtin_amdgcn_sched_barrier(0);
      gate_up_rows<LHC, RMAX>(p, TG, TU, xr, pr, rows0, lane, j, ggu, L, NoHook{});
      gate_up_compute<LHC, RMAX>(p, gs, pc, RMAX, j, TG, TU, ggu);
      IssueTile{dtile, &TD}();
    } else {
      load_tile_pair(tg, tu, lane, TG, TU);
      opaque_tile(TG);  // waits for the gate and up bytes before the down request
      opaque_tile(TU);
      IssueTile{dtile, &TD}();
      gate_up_compute<LHC, RMAX>(p, gs, pc, 0, j, TG, TU, ggu);
    }
  } else if (has_dn) {
    load_tile(dtile, lane, TD);
  }
  if (has_dn) down_compute<LIC, RMAX>(p, dslot, ds, pc, j, TD, gdn, s_h);
}

}  // namespace nvfp4moe
