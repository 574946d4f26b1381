/*
 * oracle.h - plain, slow, float64 CPU oracle for the NVFP4 MoE decode path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU library neither
 * links nor calls it, and the two share no code.
 *
 * What it computes (each function cites what it follows):
 *   - NVFP4 decode: E2M1 element codes, one E4M3 scale per 16 consecutive
 *     elements along K, one FP32 tensor scale per matrix. The Elsa RTX 5090
 *     page ("The card and the model") says the checkpoint stores the experts
 *     in 4-bit NVFP4; the element and scale encodings are the OCP MX FP4
 *     (E2M1) and OCP 8-bit E4M3 formats.
 *   - skinny products y = x W^T of a few BF16 rows with 4-bit weights (Elsa
 *     page, "Making decode faster", paragraph on skinny matrix multiplies),
 *     and with FP8 E4M3 weights under one scale per tensor ("An FP8 fast
 *     path" on the same page);
 *   - quantization of BF16 matrices to NVFP4 (amax recipe: the pages name
 *     only the tool that did it, in the "Files" list of the Qwen3.8-27B NVFP4
 *     lm_head recipe page);
 *   - the router projection (logits = x W_r^T, BF16 weights) in front of
 *     top-k routing ("The card and the model": a mixture-of-experts model);
 *   - top-k routing, grouping of (row, slot) pairs by expert, the expert
 *     feed-forward gate_up -> SiLU*up -> down, and the routing-weighted
 *     combine ("finalize" on the same page), plus an always-on shared expert
 *     kept as a separate weight-1 term ("What didn't work" on the same page:
 *     fusing it into the routed MoE gave wrong output).
 *
 * Canonical NVFP4 layout: codes uint8 [G][N][K/2], element 2b in the low
 * nibble of byte b; scales uint8 [G][N][K/16]; g float [G]. W is [N][K] and
 * y = x W^T. BF16 values are passed as raw uint16 bit patterns.
 *
 * Parity-unpinned pieces: behaviour on NaN scale codes and NaN logits (a
 * policy, not a result).
 */
#ifndef NVFP4MOE_ORACLE_H
#define NVFP4MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the products and the MoE block split their outputs over (default
 * 1). The result is bit-identical for every count: each output is computed
 * by one thread exactly as the single-threaded loop computes it. */
void oracle_set_threads(int n);
int oracle_threads(void);

double oracle_e2m1(uint32_t code);       /* code & 15 -> value */
double oracle_e4m3(uint32_t byte);       /* byte & 255 -> value, NaN for 0x7F / 0xFF */
double oracle_bf16(uint16_t bits);       /* exact widening */

/* out[G][N][K] = e2m1 * e4m3 * g in float64. */
void oracle_dequant(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t G,
                    int64_t N, int64_t K, double* out);
/* out = fl32(fl32(e2m1 * e4m3) * g): the FP32 value of a decoded weight.
 * e2m1 * e4m3 is exact in FP32, so only the multiply by g rounds. */
void oracle_dequant_f32(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t G,
                        int64_t N, int64_t K, float* out);

/* y[M][N] = sum_k x[m][k] * W[n][k], W = dequant of one matrix, float64. */
void oracle_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes,
                 const uint8_t* scales, float g, int64_t N, double* y);

/* y[M][N] = (sum_k x[m][k] * e4m3(w[n][k])) * s in float64; w FP8 E4M3 codes
 * [N][K] row-major, one scale s for the tensor. */
void oracle_gemm_fp8(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w, double s,
                     int64_t N, double* y);

/* BF16 [G][N][K] -> canonical NVFP4 (codes [G][N][K/2], scales [G][N][K/16],
 * g [G]) by the amax recipe documented in oracle.cpp; K % 16 == 0. Finite
 * inputs only (non-finite inputs: parity unpinned). */
void oracle_quantize_nvfp4(const uint16_t* x, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* scales, float* g);
uint32_t oracle_e4m3_rne(float t);  /* nearest finite E4M3 code to t >= 0, ties to even */
uint32_t oracle_e2m1_rne(float v);  /* nearest E2M1 magnitude code to v >= 0, ties to even */

/* Router projection: logits[M][E] = x W_r^T in float64; x BF16 [M][H], w_r
 * BF16 [E][H]. */
void oracle_router_logits(const uint16_t* x, int64_t M, int64_t H, const uint16_t* w_r, int64_t E,
                          double* logits);

/* Top-k routing per row: l' = fl32(l + bias) (l' = l without bias); experts
 * ordered by l' descending, ties to the lower index, NaN below -inf; ids =
 * first k in that order; w = softmax of the selected l' (float64).
 * Returns 0, or -1 if k < 1 or k > E. */
int oracle_route_topk(const float* logits, const float* bias, int64_t M, int64_t E, int64_t k,
                      int32_t* ids, double* w);

/* counts[E]; offsets[E+1] exclusive prefix sum; pairs[M*k]: for experts in
 * ascending order, the pair indices p = m*k + j with ids[p] == e, ascending;
 * active[E]: experts with counts > 0 ascending, then -1; active_offsets[E+1]:
 * offsets[active[s]] for s < n_active, M*k from there on; *n_active. */
void oracle_group_by_expert(const int32_t* ids, int64_t M, int64_t E, int64_t k, int32_t* counts,
                            int32_t* offsets, int32_t* pairs, int32_t* active,
                            int32_t* active_offsets, int32_t* n_active);

/* y[H] = W_dn (silu(u[0:I]) * u[I:2I]),  u = W_gu x,  for one BF16 row x[H]. */
void oracle_expert_ffn(const uint16_t* x, int64_t H, int64_t I, const uint8_t* gu_codes,
                       const uint8_t* gu_scales, float gu_g, const uint8_t* dn_codes,
                       const uint8_t* dn_scales, float dn_g, double* y);

/* out[m] = sum_j w[m][j] * ffn_{ids[m][j]}(x[m])  (+ ffn_shared(x[m])) (+ residual[m]).
 * Expert weights: gu [E][2I][H], dn [E][H][I] (canonical NVFP4). Shared and
 * residual pointers may be NULL. */
void oracle_moe_block(const uint16_t* x, int64_t M, int64_t H, int64_t I, int64_t E, int64_t k,
                      const int32_t* ids, const double* w, const uint8_t* gu_codes,
                      const uint8_t* gu_scales, const float* gu_g, const uint8_t* dn_codes,
                      const uint8_t* dn_scales, const float* dn_g, const uint8_t* sgu_codes,
                      const uint8_t* sgu_scales, const float* sgu_g, const uint8_t* sdn_codes,
                      const uint8_t* sdn_scales, const float* sdn_g, const uint16_t* residual,
                      double* out);

/* oracle_moe_block with the activation rows and the residual given in double
 * (any values, not only BF16 ones): the float64 chain of a layer stack runs
 * on its own unrounded output. residual may be NULL. */
void oracle_moe_block_f64(const double* x, int64_t M, int64_t H, int64_t I, int64_t E, int64_t k,
                          const int32_t* ids, const double* w, const uint8_t* gu_codes,
                          const uint8_t* gu_scales, const float* gu_g, const uint8_t* dn_codes,
                          const uint8_t* dn_scales, const float* dn_g, const uint8_t* sgu_codes,
                          const uint8_t* sgu_scales, const float* sgu_g, const uint8_t* sdn_codes,
                          const uint8_t* sdn_scales, const float* sdn_g, const double* residual,
                          double* out);

/* The whole decode step from router logits: route, group, expert FFNs,
 * combine. ids/w/out are outputs (ids [M][k], w [M][k], out [M][H]). */
int oracle_moe_decode(const uint16_t* x, const float* logits, const float* bias, int64_t M,
                      int64_t H, int64_t I, int64_t E, int64_t k, const uint8_t* gu_codes,
                      const uint8_t* gu_scales, const float* gu_g, const uint8_t* dn_codes,
                      const uint8_t* dn_scales, const float* dn_g, const uint8_t* sgu_codes,
                      const uint8_t* sgu_scales, const float* sgu_g, const uint8_t* sdn_codes,
                      const uint8_t* sdn_scales, const float* sdn_g, const uint16_t* residual,
                      int32_t* ids, double* w, double* out);

#ifdef __cplusplus
}
#endif
#endif
