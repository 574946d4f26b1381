// moe.hpp - what every MoE decode kernel shares: the call's parameters, the
// slots (one per active expert, plus the shared expert) and their rows, and
// the reduction of a tile's per-slab partial sums for a runtime row width.
//
// Tiles: with rows_per_tile(K) = 16384 / K, the gate half of one expert's
// fused [2I][H] gate_up matrix and its [H][I] down matrix both hold
// P = H * I / 16384 tiles. Slot s < n_active is expert active[s] with the
// (row, slot) pairs pairs[offsets[e] .. offsets[e+1]); slot `routed_slots` is
// the shared expert over every row.
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
  const float* gu_g;   // [E] tensor scales inside the packed gate_up tensor
  const float* dn_g;
  const float* sgu_g;
  const float* sdn_g;
  int64_t gu_mat_bytes, dn_mat_bytes;
  int M, E, k, H, I;
  int LH, LI;          // lanes per row: H / 32, I / 32
  int routed_slots, has_shared, slots;
  int P;               // tiles per gate half = tiles per down matrix = H * I / 16384
  int pair_regs;       // ceil(M * k / 64) <= 2: pairs[] is held in registers; else 0
  float* hp;           // [P_tot][I] h words (FP32, or hi / lo BF16 for MFMA slots)
  float* yp;           // [P_tot][H] expert outputs (FP32)
  int dense_min_rows;  // slots with at least this many rows use MFMA
  // optional dense projection of x, computed by the first proj_blocks blocks
  // of the down launch (token_down_combine_kernel): py [M][pn] = x W_p^T
  const uint8_t* pw;
  uint16_t* py;
  int64_t pn;
  int proj_blocks;     // a multiple of 8 (0: none), so the XCD order of the rest holds
};

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

}  // namespace nvfp4moe
