// staged.hpp - the MoE decode step in three launches, for larger row counts:
//   1. gate_up: one wave per (slot, gate tile j) writes h for the slot's rows;
//   2. down:    one wave per (slot, down tile t) writes y for the slot's rows;
//   3. combine: one thread per output, sum over slots in j order (+ shared)
//               (+ residual), rounded once to BF16.
// A launch starts after the previous one has finished, so h and y are plain
// 32-bit words: nothing is polled, nothing needs clearing, and the repeated
// reads of x and h (every tile item of a slot reads all of the slot's rows)
// are served by the L2.
//
// Slots with at least dense_min_rows rows (and the shapes the dense code
// covers: H = 2048, I = 512) use BF16 MFMA; their h words hold hi / lo BF16
// halves (dense.hpp). Other slots use the VALU tile products of tile.hpp and
// FP32 h words.
#pragma once

#include "dense.hpp"
#include "gemm.hpp"
#include "moe.hpp"

namespace nvfp4moe {

// Pair index (row of h / y) of row r of a slot, per lane; rows past the
// slot's last (padding, never written; s.rows >= 1) repeat it, so that every
// lane issues its load (see load_x_bf16).
__device__ __forceinline__ int lane_pair(const MoeParams& p, const SlotInfo& s, int r) {
  const int rc = r < s.rows ? r : s.rows - 1;
  return s.shared ? p.M * p.k + rc : p.pairs[s.row_begin + rc];
}

// Slot of a tile item: the shared expert (if any) comes first, so that its
// items, which carry every row, start with the first blocks instead of last.
__device__ __forceinline__ int staged_slot(const MoeParams& p, int item_slot) {
  if (!p.has_shared) return item_slot;
  return item_slot == 0 ? p.routed_slots : item_slot - 1;
}

// Slot of item slot `item` when the items take the slots heaviest first. With
// many rows a few popular experts hold most of them (Zipf(1.1) at M = 256: 219
// rows in one slot, whose items then take 55-75 us where a one-row item takes
// 8), and in expert order such a slot can start last and finish far behind
// the rest. Classes by row count, 1-3, 4-15, 16-63, 64-255, 256-1023, 1024 and
// up, are taken from the heaviest down, each in slot order; the shared expert
// (every row) comes first. Every wave of the launch computes the same order
// from the slots' row counts (one round trip, as slot_info's) with wave scans.
// The whole wave must be active. Returns false for items past the last slot.
__device__ __forceinline__ int row_class(int rows) {
  if (rows <= 0) return -1;
  const int c = (31 - __builtin_clz((unsigned)rows)) >> 1;
  return c < 5 ? c : 5;
}

__device__ __forceinline__ bool ordered_slot_info(const MoeParams& p, int item, SlotInfo& s) {
  const int lane = threadIdx.x & 63;
  if (p.has_shared) {
    if (item == 0) return slot_info(p, p.routed_slots, s);
    item -= 1;
  }
  // active[E] and active_offsets[E + 1] are written in full (unused slots:
  // expert -1), so every entry is read at once, without waiting for n_active
  const int E = p.E;
  int ao[5], ex[4], cls[4];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int sl = 4 * lane + j;
    const int v = p.active_offsets[sl <= E ? sl : E];
    ao[j] = sl <= E ? v : 0;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = 4 * lane + j;
    const int v = p.active[sl < E ? sl : E - 1];
    ex[j] = sl < E ? v : -1;
    cls[j] = ex[j] >= 0 ? row_class(ao[j + 1] - ao[j]) : -1;
  }
  const int cmax = (int)wave_max_u32_all((uint32_t)(max(max(cls[0], cls[1]), max(cls[2], cls[3])) + 1)) - 1;
  int base = 0;
#pragma unroll 1
  for (int c = cmax; c >= 0; --c) {
    int in[4], pos[4], total;
#pragma unroll
    for (int j = 0; j < 4; ++j) in[j] = cls[j] == c ? 1 : 0;
    wave_scan256(in, lane, pos, total);
    if (item < base + total) {
      const int rank = item - base;
      int jj = 0;
      uint64_t hit = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint64_t b = __ballot(in[j] && pos[j] == rank);
        if (b) {
          hit = b;
          jj = j;
        }
      }
      const int l = hit ? (int)__builtin_ctzll(hit) : 0;  // one lane holds the rank
      int e = 0, b0 = 0, b1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ej = __builtin_amdgcn_readlane(ex[j], l);
        const int bj = __builtin_amdgcn_readlane(ao[j], l);
        const int nj = __builtin_amdgcn_readlane(ao[j + 1], l);
        if (j == jj) {
          e = ej;
          b0 = bj;
          b1 = nj;
        }
      }
      s.e = e;
      s.row_begin = b0;
      s.rows = b1 - b0;
      s.shared = false;
      return true;
    }
    base += total;
  }
  return false;
}

template <bool ORDER>
__device__ __forceinline__ bool item_slot_info(const MoeParams& p, int item, SlotInfo& s) {
  if constexpr (ORDER) return ordered_slot_info(p, item, s);
  return slot_info(p, staged_slot(p, item), s);
}

__device__ __forceinline__ const uint8_t* gate_matrix(const MoeParams& p, const SlotInfo& s) {
  return s.shared ? p.sgu : p.gu + (int64_t)s.e * p.gu_mat_bytes;
}
__device__ __forceinline__ const uint8_t* down_matrix(const MoeParams& p, const SlotInfo& s) {
  return s.shared ? p.sdn : p.dn + (int64_t)s.e * p.dn_mat_bytes;
}

// ---- gate_up ------------------------------------------------------------------------------

// VALU: h = silu(gate) * up for R loaded rows, as FP32 words.
template <int LC, int R>
__device__ __forceinline__ void staged_gate_math(const MoeParams& p, const TileRegs& TG,
                                                 const TileRegs& TU, const uint4 (&xr)[R][4],
                                                 const int (&pr)[R], int rows, int j, float g,
                                                 int L) {
  const int lane = threadIdx.x;
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
    const int i = j * p.RH + reduced_row(lane, L);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rows) p.hp[(int64_t)pr[r] * p.I + i] = silu(ug[r] * g) * (uu[r] * g);
  }
}

// Generic row widths (any L, any number of panels), one row: h of the row's
// pair for gate row block j (gate rows in wave `gwave`'s values vg, up rows
// in vu) is written by the lanes that hold the reduced values.
__device__ __forceinline__ void write_h_generic(const MoeParams& p, int pair, int j, float g,
                                                const float (&vg)[8], const float (&vu)[8],
                                                int L) {
  const int lane = threadIdx.x & 63;
  if (!reduced_writer_rt(lane, L)) return;
  const int nv = reduced_values(L);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (q < nv)
      p.hp[(int64_t)pair * p.I + j * p.RH + reduced_row_v(lane, L, q)] =
          silu(vg[q] * g) * (vu[q] * g);
}

template <int LC, int R>
__device__ __forceinline__ void staged_gate_rows(const MoeParams& p, const SlotInfo& s,
                                                 const PairCache& c, const TileRegs& TG,
                                                 const TileRegs& TU, int r0, int rows, int j,
                                                 float g, int L) {
  int pr[R];
  uint4 xr[R][4];
  load_rows<R>(p, s, c, r0, rows, 32 * ((int)threadIdx.x % L), pr, xr);
  staged_gate_math<LC, R>(p, TG, TU, xr, pr, rows, j, g, L);
}

// The first batch of R rows: its activation rows are requested before the
// tiles, and its slabs are multiplied as they arrive (no wait for the whole
// tiles). TG / TU keep the tiles for the later batches.
template <int LC, int R>
__device__ __forceinline__ void staged_gate_first(const MoeParams& p, const SlotInfo& s,
                                                  const PairCache& c, const uint8_t* tg,
                                                  const uint8_t* tu, int rows, int j, float g,
                                                  int L, TileRegs& TG, TileRegs& TU) {
  int pr[R];
  uint4 xr[R][4];
  load_rows<R>(p, s, c, 0, rows, 32 * ((int)threadIdx.x % L), pr, xr);
  __builtin_amdgcn_sched_barrier(0);
  load_tile_pair(tg, tu, (int)threadIdx.x, TG, TU);
  __builtin_amdgcn_sched_barrier(0);
  staged_gate_math<LC, R>(p, TG, TU, xr, pr, rows, j, g, L);
}

// MFMA (H = 2048: a gate tile and an up tile hold 8 rows each, together one
// 16-row block): h packed as hi / lo BF16 for the dense down product.
// AHEAD: chunk columns of x requested ahead of the one being multiplied (a
// ring of AHEAD + 1 columns in registers; 0 in the 128-register two-wave
// kernel, where the ring costs more than it hides).
template <int NCB, int AHEAD>
__device__ __forceinline__ void staged_gate_dense(const MoeParams& p, const SlotInfo& s,
                                                  const uint8_t* tg, const uint8_t* tu, int j,
                                                  float g) {
  const int lane = threadIdx.x, m = lane & 15, grp = lane >> 4;
  DenseRows<16> d;
  {
    const int n = m;  // 0-7 gate rows, 8-15 up rows
#pragma unroll
    for (int q = 0; q < 16; ++q)
      load_dense_chunk(n < 8 ? tg : tu, 64, n & 7, 4 * q + grp, d.c[q], d.s[q]);
  }
  uint32_t* hw = reinterpret_cast<uint32_t*>(p.hp);
#pragma unroll 1
  for (int cb0 = 0; cb0 < s.rows; cb0 += 16 * NCB) {
    opaque_dense<16>(d);
    int xrow[NCB], pr[NCB];
#pragma unroll
    for (int b = 0; b < NCB; ++b) {
      const int r = cb0 + 16 * b + m;
      const int lp = lane_pair(p, s, r);
      pr[b] = r < s.rows ? lp : -1;
      xrow[b] = pair_xrow(p, lp);
    }
    f32x4 acc[NCB];
#pragma unroll
    for (int b = 0; b < NCB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (AHEAD == 0) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        bf16x8 a[4];
        dense_a<16>(d, q, a);
#pragma unroll
        for (int b = 0; b < NCB; ++b) {
          uint4 xv[4];
          load_x_bf16(p.x, p.H, xrow[b], 32 * (4 * q + grp), xv);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[b] = mfma_bf16(a[e], as_bf16x8(xv[e]), acc[b]);
        }
        __builtin_amdgcn_sched_barrier(0);  // one chunk column's loads in flight at a time
      }
    } else {
      uint4 xb[AHEAD + 1][NCB][4];
#pragma unroll
      for (int q = 0; q < AHEAD; ++q)
#pragma unroll
        for (int b = 0; b < NCB; ++b)
          load_x_bf16(p.x, p.H, xrow[b], 32 * (4 * q + grp), xb[q][b]);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (q + AHEAD < 16) {
#pragma unroll
          for (int b = 0; b < NCB; ++b)
            load_x_bf16(p.x, p.H, xrow[b], 32 * (4 * (q + AHEAD) + grp),
                        xb[(q + AHEAD) % (AHEAD + 1)][b]);
        }
        bf16x8 a[4];
        dense_a<16>(d, q, a);
#pragma unroll
        for (int b = 0; b < NCB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[b] = mfma_bf16(a[e], as_bf16x8(xb[q % (AHEAD + 1)][b][e]), acc[b]);
        __builtin_amdgcn_sched_barrier(0);  // AHEAD + 1 columns' loads in flight at most
      }
    }
    // D row 4 grp + r: gate rows 0-7 in lanes 0-31, the matching up rows in lanes 32-63
#pragma unroll
    for (int b = 0; b < NCB; ++b) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[b][r];
        const float u = partner32(v, lane);
        if (lane < 32 && pr[b] >= 0) {
          const int i = j * 8 + 4 * grp + r;
          hw[(int64_t)pr[b] * p.I + i] = pack_hilo(silu(v * g) * (u * g));
        }
      }
    }
  }
}

// ORDER: the items take the slots heaviest first (the launches for many rows).
template <int LHC, int RMAX, bool DENSE, bool ORDER>
__global__ void __launch_bounds__(64, RMAX == 1 ? 3 : 2) staged_gate_kernel(MoeParams p) {
  const int lane = threadIdx.x;
  const int j = blockIdx.x % p.PG;
  PairCache pc;
  load_pair_cache(p, lane, pc);
  SlotInfo s;
  if (!item_slot_info<ORDER>(p, blockIdx.x / p.PG, s)) return;
  const uint8_t* mat = gate_matrix(p, s);
  const float g = s.shared ? p.sgu_g[0] : p.gu_g[s.e];
  const uint8_t* tg = mat + (int64_t)j * kTileBytes;
  const uint8_t* tu = mat + (int64_t)(j + p.PG) * kTileBytes;
  if constexpr (DENSE) {
    if (s.rows >= p.dense_min_rows) {
      staged_gate_dense<2, 1>(p, s, tg, tu, j, g);
      return;
    }
  }
  const int L = LHC ? LHC : p.LH;
  if constexpr (LHC == 0) {
    if (p.QH > 1 || L < 8) {  // any row width, any number of panels: one row at a time
#pragma unroll 1
      for (int r = 0; r < s.rows; ++r) {
        const int pair = slot_pair(p, s, r, pc);
        float vg[8], vu[8];
        panels_dot_bf16<0>(mat, j, p.QH, p.KpH, p.x, p.H, pair_xrow(p, pair), lane, L, vg);
        panels_dot_bf16<0>(mat, j + p.PG, p.QH, p.KpH, p.x, p.H, pair_xrow(p, pair), lane, L,
                           vu);
        write_h_generic(p, pair, j, g, vg, vu, L);
      }
      return;
    }
  }
  TileRegs TG, TU;
  // the first batch is sized to the slot's rows (1, 2 or RMAX): the products
  // of padding rows are as dear as real ones, and most slots of a many-row
  // step hold a row or two (M = 256: three of four VALU slots)
  {
    const int rows0 = s.rows < RMAX ? s.rows : RMAX;
    if (RMAX >= 4 && rows0 > 2)
      staged_gate_first<LHC, RMAX>(p, s, pc, tg, tu, rows0, j, g, L, TG, TU);
    else if (RMAX >= 2 && rows0 == 2)
      staged_gate_first<LHC, (RMAX >= 2 ? 2 : 1)>(p, s, pc, tg, tu, rows0, j, g, L, TG, TU);
    else
      staged_gate_first<LHC, 1>(p, s, pc, tg, tu, rows0, j, g, L, TG, TU);
  }
#pragma unroll 1
  for (int r0 = RMAX; r0 < s.rows; r0 += RMAX) {
    opaque_tile(TG);
    opaque_tile(TU);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      staged_gate_rows<LHC, (RMAX >= 8 ? 8 : 1)>(p, s, pc, TG, TU, r0, rows, j, g, L);
    else if (RMAX >= 4 && rows > 2)
      staged_gate_rows<LHC, (RMAX >= 4 ? 4 : 1)>(p, s, pc, TG, TU, r0, rows, j, g, L);
    else if (RMAX >= 2 && rows > 1)
      staged_gate_rows<LHC, (RMAX >= 2 ? 2 : 1)>(p, s, pc, TG, TU, r0, rows, j, g, L);
    else
      staged_gate_rows<LHC, 1>(p, s, pc, TG, TU, r0, rows, j, g, L);
  }
}

// Gate_up with two waves per item (one row per batch): wave 0 streams the gate
// tile, wave 1 the up tile, each half the bytes and half the arithmetic of a
// one-wave item; wave 1 hands its reduced values to wave 0 through LDS.
template <int LC>
__device__ __forceinline__ float tile_row_value(const TileRegs& T, const uint4 (&xr)[1][4], int L) {
  float part[1][8];
  tile_dot_bf16<1>(T, xr, part);
  reduce_slabs_rt<LC>(part[0], (int)threadIdx.x & 63, L);
  return part[0][0];
}

// MFMA in a two-wave item for a slot of at most 16 rows (M <= 16: one pass):
// wave w takes chunk columns 8 w .. 8 w + 7, half of K. Per column it requests
// the A chunk (gate tile rows 0-7, up tile rows 0-7) and the rows' x pieces
// RING columns ahead, so a wave waits about two round trips rather than one
// per column, in few registers; wave 1 hands its partial D tile to wave 0
// through LDS, and wave 0 adds it (wave 0's half first) and writes h.
template <int RING>
__device__ __forceinline__ void staged_gate_dense_halves(const MoeParams& p, const SlotInfo& s,
                                                         const uint8_t* tg, const uint8_t* tu,
                                                         int j, float g, f32x4* dred) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 15, grp = lane >> 4;
  const bool valid = m < s.rows;
  const int pr = lane_pair(p, s, m);
  const int xrow = pair_xrow(p, pr);
  const uint8_t* tile = m < 8 ? tg : tu;
  const int q0 = 8 * wave;
  DenseRows<RING + 1> d;
  uint4 xv[RING + 1][4];
#pragma unroll
  for (int q = 0; q < RING; ++q) {
    load_dense_chunk(tile, 64, m & 7, 4 * (q0 + q) + grp, d.c[q], d.s[q]);
    load_x_bf16(p.x, p.H, xrow, 32 * (4 * (q0 + q) + grp), xv[q]);
  }
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if (q + RING < 8) {
      const int r = (q + RING) % (RING + 1);
      load_dense_chunk(tile, 64, m & 7, 4 * (q0 + q + RING) + grp, d.c[r], d.s[r]);
      load_x_bf16(p.x, p.H, xrow, 32 * (4 * (q0 + q + RING) + grp), xv[r]);
    }
    const int c = q % (RING + 1);
    bf16x8 a[4];
    dense_a<RING + 1>(d, c, a);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_bf16(a[e], as_bf16x8(xv[c][e]), acc);
    __builtin_amdgcn_sched_barrier(0);  // RING + 1 columns' loads in flight at most
  }
  if (wave == 1) dred[lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4 o = dred[lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += o[r];
    uint32_t* hw = reinterpret_cast<uint32_t*>(p.hp);
    // D row 4 grp + r: gate rows 0-7 in lanes 0-31, the matching up rows in lanes 32-63
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[r];
      const float u = partner32(v, lane);
      if (lane < 32 && valid) hw[(int64_t)pr * p.I + j * 8 + 4 * grp + r] =
          pack_hilo(silu(v * g) * (u * g));
    }
  }
}

template <int LHC, bool DENSE>
__global__ void __launch_bounds__(128, 4) staged_gate_split_kernel(MoeParams p) {
  __shared__ float up_lds[64];
  __shared__ f32x4 dred[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = staged_slot(p, blockIdx.x / p.PG), j = blockIdx.x % p.PG;
  PairCache pc;
  load_pair_cache(p, lane, pc);
  SlotInfo s;
  if (!slot_info(p, slot, s)) return;
  const uint8_t* mat = gate_matrix(p, s);
  const float g = s.shared ? p.sgu_g[0] : p.gu_g[s.e];
  const uint8_t* tg = mat + (int64_t)j * kTileBytes;
  const uint8_t* tu = mat + (int64_t)(j + p.PG) * kTileBytes;
  if constexpr (DENSE) {
    if (s.rows >= p.dense_min_rows) {
      staged_gate_dense_halves<2>(p, s, tg, tu, j, g, dred);  // s.rows <= M <= 16
      return;
    }
  }
  const int L = LHC ? LHC : p.LH;
  if constexpr (LHC == 0) {
    if (p.QH > 1 || L < 8) {  // any row width, any number of panels: wave 1 takes the up half
      __shared__ float up_rows[8][64];
      const int nv = reduced_values(L);
#pragma unroll 1
      for (int r = 0; r < s.rows; ++r) {
        const int pair = slot_pair(p, s, r, pc);
        float v[8];
        panels_dot_bf16<0>(mat, wave == 0 ? j : j + p.PG, p.QH, p.KpH, p.x, p.H,
                           pair_xrow(p, pair), lane, L, v);
        for (int q = 0; q < nv; ++q)
          if (wave == 1) up_rows[q][lane] = v[q];
        __syncthreads();
        if (wave == 0) {
          float vu[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) vu[q] = q < nv ? up_rows[q][lane] : 0.0f;
          write_h_generic(p, pair, j, g, v, vu, L);
        }
        __syncthreads();
      }
      return;
    }
  }
  const bool writer = reduced_writer_rt(lane, L);
  const int i = j * p.RH + reduced_row(lane, L);
  TileRegs T;
#pragma unroll 1
  for (int r = 0; r < s.rows; ++r) {
    int pr[1];
    uint4 xr[1][4];
    if (r == 0) {
      load_rows<1>(p, s, pc, 0, 1, 32 * (lane % L), pr, xr);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(wave == 0 ? tg : tu, lane, T);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      opaque_tile(T);
      load_rows<1>(p, s, pc, r, 1, 32 * (lane % L), pr, xr);
    }
    const float v = tile_row_value<LHC>(T, xr, L);
    if (wave == 1) up_lds[lane] = v;
    __syncthreads();
    if (wave == 0 && writer) p.hp[(int64_t)pr[0] * p.I + i] = silu(v * g) * (up_lds[lane] * g);
    __syncthreads();
  }
}

// ---- down ----------------------------------------------------------------------------------

// VALU: h rows (FP32) of R pairs.
template <int R>
__device__ __forceinline__ void staged_load_h(const MoeParams& p, const SlotInfo& s,
                                              const PairCache& c, int r0, int rows, int L,
                                              int (&pr)[R], float (&hr)[R][32]) {
  const int col0 = 32 * ((int)threadIdx.x % L);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pr[r] = r < rows ? slot_pair(p, s, r0 + r, c) : 0;
    if (r < rows) {
      load_h_f32(p.hp, p.I, pr[r], col0, hr[r]);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) hr[r][j] = 0.0f;
    }
  }
}

// VALU: y for R loaded h rows, as FP32 words.
template <int LC, int R>
__device__ __forceinline__ void staged_down_math(const MoeParams& p, const TileRegs& T,
                                                 const int (&pr)[R], const float (&hr)[R][32],
                                                 int rows, int t, float g, int L) {
  const int lane = threadIdx.x;
  float part[R][8];
  tile_dot_f32<R>(T, hr, part);
#pragma unroll
  for (int r = 0; r < R; ++r) reduce_slabs_rt<LC>(part[r], lane, L);
  const int n = t * p.RI + reduced_row(lane, L);
  if (reduced_writer_rt(lane, L) && n < p.H) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rows) p.yp[(int64_t)pr[r] * p.H + n] = part[r][0] * g;
  }
}

template <int LC, int R>
__device__ __forceinline__ void staged_down_rows(const MoeParams& p, const SlotInfo& s,
                                                 const PairCache& c, const TileRegs& T, int r0,
                                                 int rows, int t, float g, int L) {
  int pr[R];
  float hr[R][32];
  staged_load_h<R>(p, s, c, r0, rows, L, pr, hr);
  staged_down_math<LC, R>(p, T, pr, hr, rows, t, g, L);
}

// The first batch of R rows: h is complete (the gate_up launch has ended), so
// its rows go out first, then the tile, whose slabs are multiplied as they
// arrive (M = 16: 46.61 -> 46.17 us, M = 256: 208.1 -> 207.0 us).
template <int LC, int R>
__device__ __forceinline__ void staged_down_first(const MoeParams& p, const SlotInfo& s,
                                                  const PairCache& c, const uint8_t* tile,
                                                  int rows, int t, float g, int L, TileRegs& T) {
  int pr[R];
  float hr[R][32];
  staged_load_h<R>(p, s, c, 0, rows, L, pr, hr);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(tile, (int)threadIdx.x, T);
  __builtin_amdgcn_sched_barrier(0);
  staged_down_math<LC, R>(p, T, pr, hr, rows, t, g, L);
}

// MFMA (I = 512: a down tile holds 32 rows, two 16-row blocks; K = 512 is 4
// chunk columns per lane group).
template <int NCB>
__device__ __forceinline__ void staged_down_dense(const MoeParams& p, const SlotInfo& s,
                                                  const uint8_t* tile, int t, float g) {
  const int lane = threadIdx.x, m = lane & 15, grp = lane >> 4;
  DenseRows<4> d[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      load_dense_chunk(tile, 16, 16 * rb + m, 4 * q + grp, d[rb].c[q], d[rb].s[q]);
  const uint32_t* hw = reinterpret_cast<const uint32_t*>(p.hp);
#pragma unroll 1
  for (int cb0 = 0; cb0 < s.rows; cb0 += 16 * NCB) {
    opaque_dense<4>(d[0]);
    opaque_dense<4>(d[1]);
    int pr[NCB], hrow[NCB];
#pragma unroll
    for (int b = 0; b < NCB; ++b) {
      const int r = cb0 + 16 * b + m;
      hrow[b] = lane_pair(p, s, r);  // padding lanes: their D columns are not written
      pr[b] = r < s.rows ? hrow[b] : -1;
    }
    f32x4 acc[2][NCB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int b = 0; b < NCB; ++b) acc[rb][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x8 a[2][4];
      dense_a<4>(d[0], q, a[0]);
      dense_a<4>(d[1], q, a[1]);
#pragma unroll
      for (int b = 0; b < NCB; ++b) {
        // the lane's 32 h values of chunk column q (8 words per operand
        // pair), all requested before the first product that needs them
        uint4 hv[8];
        const uint4* src =
            reinterpret_cast<const uint4*>(hw + (int64_t)hrow[b] * p.I + 32 * (4 * q + grp));
#pragma unroll
        for (int v = 0; v < 8; ++v) hv[v] = src[v];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x8 hi, lo;
          split_hilo(hv[2 * e], hv[2 * e + 1], hi, lo);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            acc[rb][b] = mfma_bf16(a[rb][e], hi, acc[rb][b]);
            acc[rb][b] = mfma_bf16(a[rb][e], lo, acc[rb][b]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int b = 0; b < NCB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = t * 32 + 16 * rb + 4 * grp + r;
          if (pr[b] >= 0 && n < p.H) p.yp[(int64_t)pr[b] * p.H + n] = acc[rb][b][r] * g;
        }
  }
}

template <int LIC, int RMAX, bool DENSE, bool ORDER>
__global__ void __launch_bounds__(64, RMAX == 1 ? 3 : 2) staged_down_kernel(MoeParams p) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x % p.PD;
  PairCache pc;
  load_pair_cache(p, lane, pc);
  SlotInfo s;
  if (!item_slot_info<ORDER>(p, blockIdx.x / p.PD, s)) return;
  const uint8_t* tile = down_matrix(p, s) + (int64_t)t * kTileBytes;
  const float g = s.shared ? p.sdn_g[0] : p.dn_g[s.e];
  if constexpr (DENSE) {
    if (s.rows >= p.dense_min_rows) {
      // the M <= 16 launches (plain slot order): at most 16 rows a slot, one
      // 16-row pass
      staged_down_dense<(RMAX == 1 || !ORDER) ? 1 : 2>(p, s, tile, t, g);
      return;
    }
  }
  const int L = LIC ? LIC : p.LI;
  if constexpr (LIC == 0) {
    if (p.QI > 1 || L < 8) {  // any row width, any number of panels: one row at a time
      const int nv = reduced_values(L);
#pragma unroll 1
      for (int r = 0; r < s.rows; ++r) {
        const int pair = slot_pair(p, s, r, pc);
        float v[8];
        panels_dot_f32<0>(down_matrix(p, s), t, p.QI, p.KpI, p.hp, p.I, pair, lane, L, v);
        if (reduced_writer_rt(lane, L)) {
          for (int q = 0; q < nv; ++q) {
            const int n = t * p.RI + reduced_row_v(lane, L, q);
            if (n < p.H) p.yp[(int64_t)pair * p.H + n] = v[q] * g;
          }
        }
      }
      return;
    }
  }
  TileRegs T;
  // the first batch is sized to the slot's rows (1, 2 or RMAX), as in gate_up
  {
    const int rows0 = s.rows < RMAX ? s.rows : RMAX;
    if (RMAX >= 4 && rows0 > 2)
      staged_down_first<LIC, RMAX>(p, s, pc, tile, rows0, t, g, L, T);
    else if (RMAX >= 2 && rows0 == 2)
      staged_down_first<LIC, (RMAX >= 2 ? 2 : 1)>(p, s, pc, tile, rows0, t, g, L, T);
    else
      staged_down_first<LIC, 1>(p, s, pc, tile, rows0, t, g, L, T);
  }
#pragma unroll 1
  for (int r0 = RMAX; r0 < s.rows; r0 += RMAX) {
    opaque_tile(T);
    const int rows = (s.rows - r0) < RMAX ? (s.rows - r0) : RMAX;
    if (RMAX >= 8 && rows > 4)
      staged_down_rows<LIC, (RMAX >= 8 ? 8 : 1)>(p, s, pc, T, r0, rows, t, g, L);
    else if (RMAX >= 4 && rows > 2)
      staged_down_rows<LIC, (RMAX >= 4 ? 4 : 1)>(p, s, pc, T, r0, rows, t, g, L);
    else if (RMAX >= 2 && rows > 1)
      staged_down_rows<LIC, (RMAX >= 2 ? 2 : 1)>(p, s, pc, T, r0, rows, t, g, L);
    else
      staged_down_rows<LIC, 1>(p, s, pc, T, r0, rows, t, g, L);
  }
}

// ---- combine -------------------------------------------------------------------------------

constexpr int kMaxTopK = 8;  // the library's bound on k (checked on the host)

// One thread per output (m, n) (blocks of TPB threads, a compile-time
// constant: blockDim.x would be read from the dispatch packet before the first
// address): routed slots in j order, then shared, then
// residual. Every term's loads are issued before the first add (the loop over
// k is unrolled to its maximum), so a thread waits one round trip, not k.
template <int TPB>
__global__ void __launch_bounds__(TPB) staged_combine_kernel(MoeParams p) {
  const int64_t idx = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (idx >= (int64_t)p.M * p.H) return;
  const int m = (int)(idx / p.H), n = (int)(idx % p.H);
  float yv[kMaxTopK], wv[kMaxTopK];
#pragma unroll
  for (int t = 0; t < kMaxTopK; ++t) {
    yv[t] = 0.0f;
    wv[t] = 0.0f;
    if (t < p.k) {
      yv[t] = p.yp[((int64_t)m * p.k + t) * p.H + n];
      wv[t] = p.w[m * p.k + t];
    }
  }
  const float ys = p.has_shared ? p.yp[((int64_t)p.M * p.k + m) * p.H + n] : 0.0f;
  const float res = p.residual ? bf16_to_f32(p.residual[(int64_t)m * p.H + n]) : 0.0f;
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < kMaxTopK; ++t)
    if (t < p.k) acc += wv[t] * yv[t];
  if (p.has_shared) acc += ys;
  if (p.residual) acc += res;
  p.out[idx] = f32_to_bf16_rne(acc);
}


// ---- down + combine per row (few rows) --------------------------------------------------

// Row counts up to this take the two-launch path below by default.
constexpr int kTokenMajorMaxRows = 8;

// One block per (row m, down tile t), one wave per slot j of the row (plus one
// for the shared expert): wave j multiplies its pair's h row with tile t of
// expert ids[m][j], then the block adds the tile's outputs in j order (+ the
// shared term) (+ residual) and writes them as BF16, with the same arithmetic
// as staged_combine_kernel. With a few rows nearly every pair has its own
// expert, so reading a tile per pair rather than per expert costs almost no
// extra bytes, and y never leaves the chip (no combine launch). h must be
// FP32 words: every slot took the VALU gate_up path.
// Slot q of row m (q = k: the shared expert), down tile t: its outputs to ys[q].
// What a slot's wave requests between its tile loads and its products.
struct NoPrefetch {
  __device__ void operator()() const {}
};

// hl: the wave's LDS row for h (LIC != 0).
template <int LIC, typename Pre = NoPrefetch>
__device__ __forceinline__ void token_down_slot(const MoeParams& p, int q, int m, int t, int L,
                                                float (*ys)[LIC ? 512 / LIC : 512], uint4* hl,
                                                Pre pre = Pre()) {
  const int lane = threadIdx.x & 63;
  const bool sh = q == p.k;  // the shared expert's slot (only with has_shared)
  const int pair = sh ? p.M * p.k + m : m * p.k + q;
  const int e = sh ? 0 : p.ids[pair];
  const uint8_t* tile =
      (sh ? p.sdn : p.dn + (int64_t)e * p.dn_mat_bytes) + (int64_t)t * kTileBytes;
  const float g = sh ? p.sdn_g[0] : p.dn_g[e];
  if constexpr (LIC == 0) {
    if (p.QI > 1 || L < 8) {  // any row width, any number of panels
      pre();
      float v[8];
      panels_dot_f32<0>(sh ? p.sdn : p.dn + (int64_t)e * p.dn_mat_bytes, t, p.QI, p.KpI, p.hp,
                        p.I, pair, lane, L, v);
      if (reduced_writer_rt(lane, L))
        for (int j = 0; j < reduced_values(L); ++j) ys[q][reduced_row_v(lane, L, j)] = v[j] * g;
      return;
    }
  }
  // the tile's loads first: with h requested ahead of them (so that slabs
  // could be multiplied as they land) the step measured slower (M = 4: 15.46
  // -> 16.05 us; 40-layer stack 1226 -> 1254 us)
  TileRegs T;
  float hr[1][32];
  load_tile(tile, lane, T);
  if constexpr (LIC != 0) {
    // the pair's h row (2 KB at I = 512) in coalesced pieces through LDS
    // (with eight direct 16-byte loads per lane: M = 4 14.95 -> 14.73 us,
    // 40-layer stack 1163 -> 1135 us)
    uint4 hv[LIC / 8], hw[8];
    load_coalesced(reinterpret_cast<const uint4*>(p.hp + (int64_t)pair * p.I), lane, hv);
    pre();
    restage_row(hl, lane, lane % LIC, hv, hw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hr[0][4 * i] = __uint_as_float(hw[i].x);
      hr[0][4 * i + 1] = __uint_as_float(hw[i].y);
      hr[0][4 * i + 2] = __uint_as_float(hw[i].z);
      hr[0][4 * i + 3] = __uint_as_float(hw[i].w);
    }
  } else {
    load_h_f32(p.hp, p.I, pair, 32 * (lane % L), hr[0]);
    pre();
  }
  float part[1][8];
  tile_dot_f32<1>(T, hr, part);
  reduce_slabs_rt<LIC>(part[0], lane, L);
  if (reduced_writer_rt(lane, L)) ys[q][reduced_row(lane, L)] = part[0][0] * g;
}

template <int LIC, bool W0_SHARED>
__global__ void __launch_bounds__((kMaxTopK + 1) * 64) token_down_combine_kernel(MoeParams p) {
  __shared__ float ys[kMaxTopK + 1][LIC ? 512 / LIC : 512];  // a down tile's rows per slot
  __shared__ uint4 hls[kMaxTopK][LIC ? 8 * LIC : 1];           // each wave's h row
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < p.proj_blocks) {  // the projection's 16-row blocks of W_p (>= 4 waves)
    __shared__ f32x4 ppart[kGemmDenseWaves - 1][64];
    if ((int64_t)blockIdx.x < (tiles_per_matrix(p.pn, 2048) + 1) / 2)
      splitk_block(p.x, p.M, p.pw, p.pn, p.py, blockIdx.x, ppart);
    return;
  }
  const int b = xcd_block((int)blockIdx.x - p.proj_blocks, (int)gridDim.x - p.proj_blocks);
  // H = 2048, I = 512: 2048 / 32 down row blocks, a constant as in the
  // gate_up launch (and likewise not with the shared expert's eight waves)
  const int PD = (LIC == 16 && !W0_SHARED) ? 64 : p.PD;
  const int m = b / PD, t = b % PD;
  const int L = LIC ? LIC : p.LI;
  const int rpt = p.RI;  // output rows of a down tile
  // One wave per slot, up to eight slots. With the shared expert beside eight
  // routed ones (W0_SHARED) the block keeps eight waves and wave 0 takes the
  // shared slot first, then routed slot 0: two such blocks fit a CU, where
  // nine waves left room for one, and the shared expert's tile t, which every
  // row reads, mostly comes from cache. (40-layer stack at M = 8: nine waves
  // 1364 us; five waves of two slots each 1318 us, 1191 us after later
  // changes; eight waves with routed slot 0 first 1183 us, shared first 1180.)
  const int nrows = min(rpt, p.H - t * rpt);
  // wave 0's threads sum the first 64 output rows: their routing weights and
  // residual are requested once the wave's tile loads are out, so that they
  // are in by the barrier (before the tiles they delayed the tiles: M = 4
  // 15.43 -> 15.75 us; after them, 40-layer stack 1224.3 -> 1204.1 us)
  // (the residual load is unconditional, from x's same place without one and
  // a clamped row: under a branch the compiler waited for every load in
  // flight, the tile's included, right after it; stack 1185.3 -> 1184.4 us)
  float wv[kMaxTopK];
  uint16_t res_raw = 0;
  auto pre = [&]() {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) wv[j] = j < p.k ? p.w[m * p.k + j] : 0.0f;
    const int r = min((int)threadIdx.x, nrows - 1);
    const uint16_t* rsrc = p.residual ? p.residual : p.x;  // both [M][H]
    res_raw = rsrc[(int64_t)m * p.H + t * rpt + r];
  };
  if (wave == 0) {
    if constexpr (W0_SHARED) {
      token_down_slot<LIC>(p, p.k, m, t, L, ys, hls[0], pre);
      token_down_slot<LIC>(p, 0, m, t, L, ys, hls[0]);
    } else {
      token_down_slot<LIC>(p, 0, m, t, L, ys, hls[0], pre);
    }
  } else {
    token_down_slot<LIC>(p, wave, m, t, L, ys, hls[wave]);
  }
  __syncthreads();
  // the tile's output rows (past H in a ragged last row block: none)
  if (wave == 0 && (int)threadIdx.x < nrows) {
    const int r = (int)threadIdx.x;
    const int64_t o = (int64_t)m * p.H + t * rpt + r;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < p.k) acc += wv[j] * ys[j][r];
    if (p.has_shared) acc += ys[p.k][r];
    if (p.residual) acc += bf16_to_f32(res_raw);
    p.out[o] = f32_to_bf16_rne(acc);
  }
  for (int r = 64 + (int)threadIdx.x; r < nrows; r += (int)blockDim.x) {
    const int64_t o = (int64_t)m * p.H + t * rpt + r;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < p.k) acc += p.w[m * p.k + j] * ys[j][r];
    if (p.has_shared) acc += ys[p.k][r];
    if (p.residual) acc += bf16_to_f32(p.residual[o]);
    p.out[o] = f32_to_bf16_rne(acc);
  }
}

}  // namespace nvfp4moe
