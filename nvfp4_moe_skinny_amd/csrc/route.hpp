// route.hpp - top-k routing and grouping of (row, slot) pairs by expert.
//
// Selection is exact: every logit becomes a 32-bit key, an order-preserving
// image of the FP32 value (-0 folded onto +0, NaN below -inf). Each of k
// rounds takes the wave-wide maximum key and, among lanes holding it, the
// lowest expert index, so the k experts come out in the order a stable sort
// by (logit descending, index ascending) gives. The weights are the softmax
// over the selected logits.
// Grouping is a stable counting sort: a pair's place inside its expert's run
// is the number of earlier pairs routed to the same expert. A row's k experts
// are distinct, so up to 64 rows this count is a popcount: bit m of an
// expert's row mask says whether row m chose it, and pair (m, j) goes to the
// expert's offset plus the number of mask bits below m. More rows use ballots
// over batches of 64 pairs.
#pragma once

#include "common.hpp"

namespace nvfp4moe {

constexpr int kRouteMaxE = 256;
constexpr int kRouteMaxK = 8;
constexpr int kRouteWaves = 16;          // 1024 threads
constexpr int kRouteSingleBlockRows = 64;  // rows routed and grouped in one launch

// Order-preserving image of an FP32 logit: larger logit -> larger key; -0
// and +0 map together; NaN maps to 1, below -inf (0x007FFFFF); 0 marks an
// empty or already-selected slot.
__device__ __forceinline__ uint32_t route_ord(float l) {
  uint32_t b = __float_as_uint(l);
  if (b == 0x80000000u) b = 0u;
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return 1u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Sum of lanes 0..15 (the others may hold anything), returned uniform.
__device__ __forceinline__ float row0_sum(float v) {
  v += __uint_as_float(dpp_u32(__float_as_uint(v), kDppQuadXor1));
  v += __uint_as_float(dpp_u32(__float_as_uint(v), kDppQuadXor2));
  v += __uint_as_float(dpp_u32(__float_as_uint(v), kDppRowRor4));
  v += __uint_as_float(dpp_u32(__float_as_uint(v), kDppRowRor8));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
}

// Requests a row's logits and bias for the experts lane + 64 s (one round
// trip; nothing waits here). Unconditional loads: without a bias the second
// set reads the row's logits again and goes unused. In the single-launch
// routing kernel this measured faster than skipping them (router + top-k at
// M=4 6.53 -> 6.12 us); the per-row kernels keep the skip (route_row_core).
__device__ __forceinline__ void route_fetch(const float* __restrict__ logits,
                                            const float* __restrict__ bias, int E, int row,
                                            int lane, float (&lv)[4], float (&bv)[4]) {
  const float* lrow = logits + (int64_t)row * E;
  const float* bsrc = bias ? bias : lrow;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    const int ec = e < E ? e : E - 1;  // in bounds; masked below
    lv[s] = lrow[ec];
    bv[s] = bsrc[ec];
  }
}

// Selects from a row's logits lv and bias bv (as route_fetch lays them out;
// bv unused without a bias) with one wave (the whole wave active): lane j < k
// returns the j-th selected expert in my_id and its weight in my_w. Each round
// takes the largest remaining key; among equal keys the ballots pick the
// lowest expert index (e = lane + 64 s). lp: E floats of LDS owned by the wave.
__device__ __forceinline__ void route_select(const float (&lv)[4], const float (&bv)[4],
                                             const float* bias, int E, int k,
                                             int lane, float* lp, int& my_id_out, float& my_w,
                                             int rounds = kRouteMaxK, bool weights = true) {
  uint32_t ord[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    const float l = bias ? lv[s] + bv[s] : lv[s];
    if (e < E) lp[e] = l;
    ord[s] = e < E ? route_ord(l) : 0u;
  }
  int my_id = 0;
  const int nr = rounds < k ? rounds : k;  // the first nr experts only (weights need all k)
  for (int j = 0; j < nr; ++j) {
    const uint32_t best = wave_max_u32_all(max(max(ord[0], ord[1]), max(ord[2], ord[3])));
    const uint64_t b0 = __ballot(ord[0] == best), b1 = __ballot(ord[1] == best);
    const uint64_t b2 = __ballot(ord[2] == best), b3 = __ballot(ord[3] == best);
    const int e = b0 ? (int)__builtin_ctzll(b0)
                     : b1 ? 64 + (int)__builtin_ctzll(b1)
                          : b2 ? 128 + (int)__builtin_ctzll(b2) : 192 + (int)__builtin_ctzll(b3);
    const bool mine = lane == (e & 63);
    const int se = e >> 6;
#pragma unroll
    for (int s = 0; s < 4; ++s) ord[s] = (mine && se == s) ? 0u : ord[s];
    my_id = lane == j ? e : my_id;
  }
  my_id_out = my_id;
  my_w = 0.0f;
  if (!weights) return;
  __builtin_amdgcn_wave_barrier();
  const float top = lp[__builtin_amdgcn_readfirstlane(my_id)];
  const float ex = lane < k ? expf(lp[my_id] - top) : 0.0f;
  const float z = row0_sum(ex);
  my_w = ex / z;
}

// Loads and selects one row. The bias loads are skipped without a bias: in
// the fused gate_up kernel, whose waves also have their activation row in
// flight, that measured faster than route_fetch's form (M=4 15.45 against
// 15.63 us per step, 40-layer stack 1226 against 1248 us).
__device__ __forceinline__ void route_row_core(const float* __restrict__ logits,
                                               const float* __restrict__ bias, int E, int k,
                                               int row, int lane, float* lp, int& my_id,
                                               float& my_w, int rounds = kRouteMaxK,
                                               bool weights = true) {
  float lv[4], bv[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    const int ec = e < E ? e : E - 1;  // in bounds; masked below
    lv[s] = logits[(int64_t)row * E + ec];
    bv[s] = bias ? bias[ec] : 0.0f;
  }
  route_select(lv, bv, bias, E, k, lane, lp, my_id, my_w, rounds, weights);
}

// Routes one row with one wave: ids and weights to global memory.
__device__ __forceinline__ void route_row(const float* __restrict__ logits,
                                          const float* __restrict__ bias, int E, int k, int row,
                                          int lane, float* lp, int32_t* __restrict__ ids,
                                          float* __restrict__ w) {
  int my_id;
  float my_w;
  route_row_core(logits, bias, E, k, row, lane, lp, my_id, my_w);
  if (lane < k) {
    ids[(int64_t)row * k + lane] = my_id;
    w[(int64_t)row * k + lane] = my_w;
  }
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts by 1, 2, 4 and 8
// within each 16-lane row, then lane 15 of a row into the next row and lane
// 31 into the upper two rows (lanes shifted in from outside a row add 0).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
  return v;
}

// Inclusive scan over 256 entries held 4 per lane (lane l: entries 4l..4l+3)
// by one wave; returns the exclusive prefix of each entry in ex[4].
__device__ __forceinline__ void wave_scan256(const int (&v)[4], int lane, int (&ex)[4], int& total) {
  const int s0 = v[0], s1 = s0 + v[1], s2 = s1 + v[2], s3 = s2 + v[3];
  const int incl = wave_inclusive_scan(s3);
  const int base = incl - s3;
  ex[0] = base;
  ex[1] = base + s0;
  ex[2] = base + s1;
  ex[3] = base + s2;
  total = __builtin_amdgcn_readlane(incl, 63);
  (void)lane;
}

// Lanes of this wave whose expert id equals this lane's (among `valid`
// lanes), from one ballot per bit of the 8-bit id.
__device__ __forceinline__ uint64_t match_id(int e, bool valid) {
  uint64_t mask = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t B = __ballot(bit);
    mask &= bit ? B : ~B;
  }
  return valid ? mask : 0ull;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// From the pair count of every expert (lane l: experts 4l .. 4l + 3), by one
// wave: each expert's run start (run_lds, and offsets), its count, and the
// active slots in expert order (then -1 with the total as offset up to E).
__device__ __forceinline__ void write_runs(const int (&c)[4], int E, int lane, int* run_lds,
                                           int32_t* __restrict__ counts,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ active,
                                           int32_t* __restrict__ active_offsets,
                                           int32_t* __restrict__ n_active) {
  int f[4], cex[4], fex[4], ctot, ftot;
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = c[j] > 0 ? 1 : 0;
  wave_scan256(c, lane, cex, ctot);
  wave_scan256(f, lane, fex, ftot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    run_lds[e] = cex[j];
    if (e < E) {
      counts[e] = c[j];
      offsets[e] = cex[j];
      if (f[j]) {  // active slots [0, ftot)
        active[fex[j]] = e;
        active_offsets[fex[j]] = cex[j];
      }
      if (e >= ftot) {  // unused slots [ftot, E)
        active[e] = -1;
        active_offsets[e] = ctot;
      }
    }
  }
  if (lane == 0) {
    offsets[E] = ctot;
    active_offsets[E] = ctot;
    *n_active = ftot;
  }
}

// Single-launch routing for M <= kRouteSingleBlockRows: one block of 16
// waves, a wave per row. Each routed row sets its bit in the row masks of its
// k experts (LDS atomic OR: the result does not depend on the order), wave 0
// turns the masks' popcounts into runs, and every thread places pairs.
__global__ void __launch_bounds__(1024) route_group_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int M, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pairs, int32_t* __restrict__ active,
    int32_t* __restrict__ active_offsets, int32_t* __restrict__ n_active) {
  __shared__ float lp[kRouteWaves][kRouteMaxE];
  __shared__ int32_t ids_lds[kRouteSingleBlockRows * kRouteMaxK];
  __shared__ unsigned long long rows_lds[kRouteMaxE];  // bit m: row m chose the expert
  __shared__ int run_lds[kRouteMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float lv[4], bv[4];
  if (wave < M) route_fetch(logits, bias, E, wave, lane, lv, bv);  // before the barrier
  if (threadIdx.x < kRouteMaxE) rows_lds[threadIdx.x] = 0ull;
  __syncthreads();
  for (int row = wave; row < M; row += kRouteWaves) {
    if (row != wave) route_fetch(logits, bias, E, row, lane, lv, bv);
    int my_id;
    float my_w;
    route_select(lv, bv, bias, E, k, lane, lp[wave], my_id, my_w);
    if (lane < k) {
      ids[(int64_t)row * k + lane] = my_id;
      w[(int64_t)row * k + lane] = my_w;
      ids_lds[row * k + lane] = my_id;
      atomicOr(&rows_lds[my_id], 1ull << row);
    }
  }
  __syncthreads();
  if (wave == 0) {
    int c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __popcll(rows_lds[4 * lane + j]);
    write_runs(c, E, lane, run_lds, counts, offsets, active, active_offsets, n_active);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < M * k; p += blockDim.x) {
    const int e = ids_lds[p];
    const int row = p / k;
    pairs[run_lds[e] + __popcll(rows_lds[e] & lanes_below(row))] = p;
  }
}

// Larger M, first launch: one wave per row, four rows a block, so that the
// rows spread over the compute units (M = 256: 64 units instead of 16, 206.6
// -> 205.9 us per step; one or two rows a block measured the same).
constexpr int kRowWaves = 4;
__global__ void __launch_bounds__(kRowWaves * 64)
route_rows_kernel(const float* __restrict__ logits, const float* __restrict__ bias, int M, int E,
                  int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float lp[kRowWaves][kRouteMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowWaves + wave;
  if (row < M) route_row(logits, bias, E, k, row, lane, lp[wave], ids, w);
}

// Larger M, second launch, up to kGroupMaskRows rows: the row masks of
// route_group_kernel with kGroupMaskRows / 64 words per expert, one block.
// Every thread takes up to eight pairs: it sets their rows' bits (LDS atomic
// OR), a thread per expert turns the words' popcounts into the number of
// earlier rows before each word, wave 0 writes the runs, and every thread
// places its pairs. The same pairs, bit for bit, as the ballot sort below.
constexpr int kGroupMaskRows = 1024;
constexpr int kGroupMaskWords = kGroupMaskRows / 64;
__global__ void __launch_bounds__(1024) group_rows_kernel(const int32_t* __restrict__ ids,
                                                          int M, int E, int k,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ pairs,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ active_offsets,
                                                          int32_t* __restrict__ n_active) {
  __shared__ unsigned long long rows_lds[kRouteMaxE][kGroupMaskWords];  // bit: row chose e
  __shared__ int below_lds[kRouteMaxE][kGroupMaskWords];  // rows of e in the words before
  __shared__ int run_lds[kRouteMaxE];
  __shared__ int cnt_lds[kRouteMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = M * k, W = (M + 63) / 64;
  int my_e[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {  // the ids first (one round trip)
    const int q = (int)threadIdx.x + u * 1024;
    my_e[u] = q < P ? ids[q] : -1;
  }
  for (int i = (int)threadIdx.x; i < kRouteMaxE * kGroupMaskWords; i += 1024)
    (&rows_lds[0][0])[i] = 0ull;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (my_e[u] >= 0) {
      const int row = ((int)threadIdx.x + u * 1024) / k;
      atomicOr(&rows_lds[my_e[u]][row >> 6], 1ull << (row & 63));
    }
  }
  __syncthreads();
  if (threadIdx.x < kRouteMaxE) {
    const int e = (int)threadIdx.x;
    int run = 0;
    for (int wd = 0; wd < W; ++wd) {
      below_lds[e][wd] = run;
      run += __popcll(rows_lds[e][wd]);
    }
    cnt_lds[e] = run;
  }
  __syncthreads();
  if (wave == 0) {
    int c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = cnt_lds[4 * lane + j];
    write_runs(c, E, lane, run_lds, counts, offsets, active, active_offsets, n_active);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = my_e[u];
    if (e >= 0) {
      const int q = (int)threadIdx.x + u * 1024;
      const int row = q / k, wd = row >> 6;
      const int before = below_lds[e][wd] + __popcll(rows_lds[e][wd] & lanes_below(row & 63));
      pairs[run_lds[e] + before] = q;
    }
  }
}

// Larger M, second launch: group all pairs in one block (P <= kGroupMaxPairs)
// with all 16 waves: the same stable counting sort, with the pairs cut into
// 16 consecutive chunks. Each wave counts its chunk per expert; a thread per
// expert turns the 16 counts into the chunks' starting places within the
// expert's run (a prefix over the waves, so earlier chunks come first); wave 0
// scans the totals into offsets and slots; then every wave places its chunk,
// batch by batch, as the one-wave sort does.
constexpr int kGroupMaxPairs = 8192;
__global__ void __launch_bounds__(1024) group_kernel(const int32_t* __restrict__ ids, int M, int E,
                                                     int k, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ pairs,
                                                     int32_t* __restrict__ active,
                                                     int32_t* __restrict__ active_offsets,
                                                     int32_t* __restrict__ n_active) {
  __shared__ int32_t ids_lds[kGroupMaxPairs];
  __shared__ int wcnt[kRouteWaves][kRouteMaxE];  // counts, then run positions, per wave
  __shared__ int total[kRouteMaxE];
  __shared__ int start[kRouteMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = M * k;
  const int chunk = ((P + kRouteWaves - 1) / kRouteWaves + 63) / 64 * 64;
  const int p_begin = wave * chunk;
  const int p_end = p_begin + chunk < P ? p_begin + chunk : P;
  for (int p = threadIdx.x; p < P; p += blockDim.x) ids_lds[p] = ids[p];
#pragma unroll
  for (int j = 0; j < 4; ++j) wcnt[wave][4 * lane + j] = 0;
  __syncthreads();
  // counts of this wave's chunk
  for (int p0 = p_begin; p0 < p_end; p0 += 64) {
    const bool valid = p0 + lane < p_end;
    const int e = valid ? ids_lds[p0 + lane] : 0;
    const uint64_t same = match_id(e, valid);
    if (valid && (same & lanes_below(lane)) == 0) wcnt[wave][e] += __popcll(same);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // per expert: chunk places relative to the expert's run start, and the total
  if (threadIdx.x < kRouteMaxE) {
    const int e = threadIdx.x;
    int run = 0;
    for (int w2 = 0; w2 < kRouteWaves; ++w2) {
      const int c = wcnt[w2][e];
      wcnt[w2][e] = run;
      run += c;
    }
    total[e] = run;
  }
  __syncthreads();
  if (wave == 0) {
    int c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = total[4 * lane + j];
    write_runs(c, E, lane, start, counts, offsets, active, active_offsets, n_active);
  }
  __syncthreads();
  // places of this wave's chunk
#pragma unroll
  for (int j = 0; j < 4; ++j) wcnt[wave][4 * lane + j] += start[4 * lane + j];
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  for (int p0 = p_begin; p0 < p_end; p0 += 64) {
    const bool valid = p0 + lane < p_end;
    const int e = valid ? ids_lds[p0 + lane] : 0;
    const uint64_t same = match_id(e, valid);
    if (valid) {
      const uint64_t below = same & lanes_below(lane);
      pairs[wcnt[wave][e] + __popcll(below)] = p0 + lane;
      if (below == 0) wcnt[wave][e] += __popcll(same);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace nvfp4moe
