// moe.hpp - what every MoE decode kernel shares: the call's parameters, the
// slots (one per active expert, plus the shared expert) and their rows, and
// the reduction of a tile's per-slab partial sums for a runtime row width.
//
// Row blocks: the gate half of one expert's fused [2I][H] gate_up matrix
// holds PG = I / RH row blocks of RH = 16384 / panel_k(H) rows (the up half
// the next PG), each of QH = H / panel_k(H) tiles; its [H][I] down matrix
// holds PD = ceil(H / RI) row blocks of RI = 16384 / panel_k(I) rows, each of
// QI tiles. With H = 2048 and I = 512 (one panel each) PG = PD = 64 and a
// row block is one tile. Slot s < n_active is expert active[s] with the
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
  int LH, LI;          // lanes per row of a panel: panel_k(H) / 32, panel_k(I) / 32
  int QH, QI;          // panels: H / panel_k(H), I / panel_k(I)
  int KpH, KpI;        // panel widths
  int RH, RI;          // rows per tile: 16384 / panel_k(H), 16384 / panel_k(I)
  int PG;              // row blocks per gate (or up) half: I / RH
  int PD;              // row blocks of a down matrix: ceil(H / RI)
  int routed_slots, has_shared, slots;
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
  for (int q = 0; q < 2; ++q) {
    const int idx = q * 64 + lane;
    c.v[q] = p.pairs[idx < n ? idx : n - 1];  // read only below n, and only if pair_regs
  }
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

// ---- segmented reduction with a runtime row width -------------------------------------

__device__ __forceinline__ int log2i(int v) { return 31 - __builtin_clz(v); }

// Reduces a lane's 8 per-slab partial sums over the L lanes that share a row
// (L = LC when LC != 0, else the runtime Lrt; L a power of two <= 64). After:
// L >= 8: v[0] holds the full sum of slab ((l & (L-1)) >> (log2 L - 3)),
// identical in the L/8 lanes of its group; L < 8: v[0 .. 8/L) hold the sums
// of slabs ((l & (L-1)) << (3 - log2 L)) + j. reduced_values / reduced_row_v
// / reduced_writer_rt name them.
template <int LC>
__device__ __forceinline__ void reduce_slabs_rt(float (&v)[8], int lane, int Lrt) {
  if constexpr (LC != 0) {
    reduce_slabs<LC>(v, lane);
  } else {
    const int halvings = Lrt >= 8 ? 3 : log2i(Lrt);
    int count = 8;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      if (t < halvings) {
        const int d = Lrt >> (t + 1);
        const int half = count >> 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < half) v[j] = halve(v[j], v[j + half], d, lane);
        }
        count = half;
      }
    }
    for (int d = Lrt / 16; d >= 1; d >>= 1) v[0] = fold(v[0], d, lane);
  }
}

// Reduced values per lane: 1 for L >= 8, else 8 / L.
__device__ __forceinline__ int reduced_values(int L) { return L >= 8 ? 1 : 8 / L; }

// Tile row of reduced value j of `lane`.
__device__ __forceinline__ int reduced_row_v(int lane, int L, int j) {
  const int slab = L >= 8 ? ((lane & (L - 1)) >> (log2i(L) - 3)) & 7
                          : ((lane & (L - 1)) << (3 - log2i(L))) + j;
  return slab * (64 / L) + lane / L;
}
__device__ __forceinline__ int reduced_row(int lane, int L) { return reduced_row_v(lane, L, 0); }

// Lanes that write their reduced values (one per distinct result).
__device__ __forceinline__ bool reduced_writer_rt(int lane, int L) {
  return L <= 8 || (lane & (L / 8 - 1)) == 0;
}

// ---- a row block over its panels, one activation row ------------------------------------

// v = the per-slab sums of row block rb of a matrix (its Q tiles back to back
// from `mat`) with one activation row, reduced over the row's lanes
// (reduce_slabs_rt): BF16 row x[xrow] of length ldx, or FP32 row h[hrow].
// Each panel's tile and the row's matching columns are loaded in turn.
template <int LC>
__device__ __forceinline__ void panels_dot_bf16(const uint8_t* mat, int rb, int Q, int Kp,
                                                const uint16_t* x, int64_t ldx, int64_t xrow,
                                                int lane, int L, float (&v)[8]) {
  float acc[1][8] = {{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll 1
  for (int q = 0; q < Q; ++q) {
    uint4 xr[1][4];
    load_x_bf16(x, ldx, xrow, q * Kp + 32 * (lane % L), xr[0]);
    TileRegs T;
    load_tile(mat + ((int64_t)rb * Q + q) * kTileBytes, lane, T);
    tile_dot_bf16<1, true>(T, xr, acc);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = acc[0][i];
  reduce_slabs_rt<LC>(v, lane, L);
}

template <int LC>
__device__ __forceinline__ void panels_dot_f32(const uint8_t* mat, int rb, int Q, int Kp,
                                               const float* h, int64_t ldh, int64_t hrow,
                                               int lane, int L, float (&v)[8]) {
  float acc[1][8] = {{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll 1
  for (int q = 0; q < Q; ++q) {
    float hr[1][32];
    load_h_f32(h, ldh, hrow, q * Kp + 32 * (lane % L), hr[0]);
    TileRegs T;
    load_tile(mat + ((int64_t)rb * Q + q) * kTileBytes, lane, T);
    tile_dot_f32<1, true>(T, hr, acc);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = acc[0][i];
  reduce_slabs_rt<LC>(v, lane, L);
}

// Pair ids and activation rows r0 .. r0 + R - 1 of a slot (rows past `rows`:
// zeros, not loaded; `rows` is the same in every lane, so the branch is the
// wave's, and the batch's products wait for every load of it anyway).
template <int R>
__device__ __forceinline__ void load_rows(const MoeParams& p, const SlotInfo& s,
                                          const PairCache& c, int r0, int rows, int col0,
                                          int (&pr)[R], uint4 (&xr)[R][4]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r, c) : 0;
    if (r < rows) {
      load_x_bf16(p.x, p.H, pair_xrow(p, pr[r]), col0, xr[r]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[r][j] = make_uint4(0, 0, 0, 0);
    }
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
