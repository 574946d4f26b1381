/*
 * nvfp4moe.h - C ABI of libnvfp4moe.so: the decode-time mixture-of-experts
 * contraction on 4-bit NVFP4 weights, for AMD Instinct MI355X (gfx950).
 *
 * The operation. In decode, most products are skinny: a handful of BF16
 * activation rows times a large 4-bit weight matrix (Elsa RTX 5090 page,
 * "Making decode faster", skinny matrix multiplies; there the 4-bit weights
 * are used with 16-bit activations). A few token rows are routed top-k to
 * experts stored in NVFP4 (same page, "The card and the model"), pushed
 * through gate_up -> SiLU*up -> down and combined with the routing weights
 * (the "finalize" step of the same page's "One environment variable"). An
 * always-on shared expert is a separate weight-1 term ("What didn't work":
 * fusing it into the routed MoE gave wrong output). Each step reads every
 * touched expert weight once, so it is bounded by memory bandwidth (the
 * decode roofline of the "One config is the weakest card's config" page,
 * "The numbers").
 *
 * NVFP4, canonical form (what callers hold):
 *   codes  uint8 [G][N][K/2]  E2M1 element codes (OCP MX FP4); element 2b of a
 *                             row is the low nibble of byte b, 2b+1 the high
 *   scales uint8 [G][N][K/16] E4M3 scale (OCP FP8 E4M3, no infinities) per 16
 *                             consecutive elements along K
 *   g      float [G]          FP32 tensor scale per matrix
 *   weight W[n][k] = e2m1(code) * e4m3(scale[n][k/16]) * g; a matrix is
 *   [N][K] (out x in) and is applied as y = x W^T.
 *
 * Conventions for every call:
 *   - Status: 0 = NVFP4MOE_OK, negative = error (codes below). On error
 *     nothing is launched; nvfp4moe_last_error_detail() says why.
 *   - All array pointers are DEVICE pointers unless stated otherwise. The
 *     caller owns all memory. The library never allocates, frees,
 *     synchronises or copies to the host, so every call is stream-ordered on
 *     the given hipStream_t (NULL = default stream) and may be captured in a
 *     HIP graph.
 *   - Arguments are validated on the host before launch. Faults inside a
 *     kernel (for example from a bad device pointer) surface at the caller's
 *     next synchronisation.
 *   - Shapes are int64_t. Support set: K % 32 == 0 with 32 <= K <= 65536; N >= 1;
 *     1 <= k <= 8; 1 <= E <= 256. Anything else returns
 *     NVFP4MOE_ERR_UNSUPPORTED; no shape ever falls back to another path.
 *   - Stateless and thread-safe.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4MOE_OK 0
#define NVFP4MOE_ERR_NULL_ARG (-1)
#define NVFP4MOE_ERR_BAD_SHAPE (-2)
#define NVFP4MOE_ERR_UNSUPPORTED (-3)
#define NVFP4MOE_ERR_WORKSPACE (-4)
#define NVFP4MOE_ERR_HIP (-5)

/* Name of a status code; never NULL. */
const char* nvfp4moe_strerror(int32_t status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* nvfp4moe_last_error_detail(void);
/* Library version string. */
const char* nvfp4moe_version(void);

/* ---- weight layout ------------------------------------------------------------
 *
 * The library streams weights in its own packed layout: a lossless byte
 * permutation of the canonical form that puts each wavefront's codes and
 * scales in 1 KB contiguous runs (the columns in panels of the largest
 * 32 * 2^j <= 2048 dividing K; its size is a whole number of 9216-byte tiles
 * per 16384 / panel rows, plus the tensor scales). The packed layout is
 * opaque: to take a slice of a matrix, slice the canonical form and pack
 * again (slicing a repacked 4-bit head silently produced garbage on the Elsa
 * page, "FR-Spec, and a silent bug").
 */

/* Bytes of packed storage for G matrices of N x K. Returns < 0 (an error
 * code) for an unsupported K or a non-positive size. */
int64_t nvfp4_packed_bytes(int64_t G, int64_t N, int64_t K);

/* Canonical -> packed. codes [G][N][K/2], scales [G][N][K/16], g [G] (all
 * device memory); packed receives nvfp4_packed_bytes(G, N, K) bytes. Rows
 * beyond N inside the last tile are zero-filled. */
int32_t nvfp4_pack(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t G,
                   int64_t N, int64_t K, void* packed, hipStream_t stream);

/* Decodes a packed tensor back to FP32 with the same device decode routines
 * the products use: out[G][N][K] = fl32(fl32(e2m1 * e4m3) * g) (apply_g != 0)
 * or e2m1 * e4m3 (apply_g == 0; exact). path selects the element decoder:
 * 0 = the BF16 pair decoder of the activation-row products, 1 = the FP32
 * pair decoder of the FP32-row products. Test hook for bit-exact decode. */
int32_t nvfp4_dequant_f32(const void* packed, int64_t G, int64_t N, int64_t K, int32_t apply_g,
                          int32_t path, float* out, hipStream_t stream);

/* ---- quantization ------------------------------------------------------------------
 *
 * BF16 matrices x [G][N][K] (raw bits) -> canonical NVFP4: codes [G][N][K/2]
 * (element 2b in the low nibble of byte b), E4M3 scales [G][N][K/16], FP32
 * tensor scales g [G]; nvfp4_pack then gives the library layout. The pages
 * name only the tool that quantized a BF16 head (the Qwen3.8-27B NVFP4 lm_head
 * recipe page, "Files": its lm_head quantization script), not its recipe;
 * this is the plain amax recipe, every division and product in FP32:
 *   g[i] = amax_i / 2688 (6 * 448), or 1 when matrix i is all zeros;
 *   scale of a 16-block = E4M3 nearest to amax_b / (6 g), ties to the even
 *     code, saturating at 448;
 *   code = sign(x) | E2M1 nearest to |x| / (scale * g), ties to the even
 *     code, saturating at 6; magnitude 0 where scale * g = 0.
 * Finite inputs (non-finite inputs give unspecified codes). g is used as
 * scratch for the per-matrix maxima between the launches (four on `stream`).
 * K % 16 == 0, G <= 65535; x 16-byte, codes 8-byte, g 4-byte aligned. */
int32_t nvfp4_quantize(const uint16_t* x, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                       uint8_t* scales, float* g, hipStream_t stream);

/* ---- dense skinny product ----------------------------------------------------------
 *
 * y[M][N] = bf16_rne( sum_k x[m][k] * W[n][k] ), one packed matrix (G = 1),
 * FP32 accumulation, BF16 activations x [M][K] and output y [M][N] (raw BF16
 * bits). M >= 1, N >= 1, K % 32 == 0 with 32 <= K <= 65536 (else
 * NVFP4MOE_ERR_UNSUPPORTED); x and w_packed 16-byte aligned. The FP32
 * summation order depends on the shape: VALU tile products (rows in batches
 * of 8; with several panels, each panel's partial sums added in panel order
 * before the reduction over lanes) for M < 4 or K != 2048;
 * BF16 MFMA tiles (the weights decode exactly to BF16) for K = 2048 and
 * M >= 4, with K split over four waves when M <= 16 and N <= 4096.
 */
int32_t nvfp4_skinny_gemm(const uint16_t* x, int64_t M, int64_t K, const void* w_packed,
                          int64_t N, uint16_t* y, hipStream_t stream);

/* ---- FP8 skinny product -------------------------------------------------------------
 *
 * y[M][N] = bf16_rne( (sum_k x[m][k] * W[n][k]) * scale[0] ), W an FP8 E4M3
 * ("FN": bias 7, max 448, 0x7F / 0xFF NaN) matrix [N][K] stored row-major as
 * bytes (used as stored: no packing step), one FP32 scale for the whole
 * tensor (a device pointer, so that the call can be graph-captured), FP32
 * accumulation. The attention projections of the pages' model are of this
 * kind (Elsa page, "An FP8 fast path": a small-batch FP8 GEMM with one scale per
 * tensor). x [M][K] and y [M][N] are raw BF16 bits; M >= 1 (taken in batches
 * of 4 rows over the same weight registers), N >= 1, K in {1024, 2048, 4096}
 * (else NVFP4MOE_ERR_UNSUPPORTED); x and W 16-byte aligned.
 */
int32_t fp8_skinny_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w_fp8,
                        const float* scale, int64_t N, uint16_t* y, hipStream_t stream);

/* ---- routing -------------------------------------------------------------------------
 *
 * Per row m: l'[e] = fl32(logits[m][e] + bias[e]) (bias may be NULL: l' =
 * logits); experts ordered by l' descending, ties to the lower expert index,
 * +0 == -0, NaN after -inf; ids[m][0..k) = the first k in that order;
 * w[m][j] = exp(l'_j - l'_0) / sum_i exp(l'_i - l'_0) over the selected
 * (FP32, sums to 1). Then the (row, slot) pairs p = m*k + j are grouped by
 * expert:
 *   counts[E]      pairs per expert
 *   offsets[E+1]   exclusive prefix sum of counts
 *   pairs[M*k]     for experts in ascending order, their p ascending
 *   active[E]      experts with counts > 0 in ascending order ("slots"), then -1
 *   active_offsets[E+1]  where each slot's run starts in pairs:
 *                  offsets[active[s]] for s < n_active, M*k from there on
 *   n_active[1]    number of slots
 * All outputs are device memory and are never read back, so the call can be
 * captured. logits [M][E] FP32, bias [E] FP32. */
int32_t moe_route_topk(const float* logits, const float* bias, int64_t M, int64_t E, int64_t k,
                       int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* pairs,
                       int32_t* active, int32_t* active_offsets, int32_t* n_active,
                       hipStream_t stream);

/* Router projection, then the routing above: logits[m][e] = sum_h x[m][h] *
 * w_router[e][h] with FP32 accumulation and FP32 result, written to the
 * caller's logits buffer [M][E] (an output: it is also what the selection
 * reads), then exactly moe_route_topk(logits, bias, ...). The pages' model is
 * a routed mixture of experts (Elsa page, "The card and the model"); its router
 * is neither an NVFP4 expert nor an FP8 projection, so w_router is BF16 [E][H]
 * (raw bits) and x is BF16 [M][H]. H in {512, 1024, 2048, 4096} (else
 * NVFP4MOE_ERR_UNSUPPORTED); x and w_router 16-byte aligned; the limits on M,
 * E and k are those of moe_route_topk. Two or three launches on `stream`. */
int32_t moe_route_project_topk(const uint16_t* x, const uint16_t* w_router, const float* bias,
                               int64_t M, int64_t E, int64_t k, int64_t H, float* logits,
                               int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* pairs, int32_t* active, int32_t* active_offsets,
                               int32_t* n_active, hipStream_t stream);

/* ---- MoE block -------------------------------------------------------------------------- */

typedef struct moe_nvfp4_args {
  const uint16_t* x;          /* [M][H] BF16 activation rows */
  const int32_t* ids;         /* [M][k]   from moe_route_topk */
  const float* w;             /* [M][k]   from moe_route_topk */
  const int32_t* offsets;     /* [E+1]    from moe_route_topk */
  const int32_t* pairs;       /* [M*k]    from moe_route_topk */
  const int32_t* active;      /* [E]      from moe_route_topk */
  const int32_t* active_offsets; /* [E+1] from moe_route_topk */
  const int32_t* n_active;    /* [1]      from moe_route_topk */
  const void* w_gate_up;      /* packed G = E, N = 2I, K = H; rows 0..I-1 gate, I..2I-1 up */
  const void* w_down;         /* packed G = E, N = H, K = I */
  const void* shared_gate_up; /* packed G = 1, N = 2I, K = H, or NULL (no shared expert) */
  const void* shared_down;    /* packed G = 1, N = H, K = I, or NULL */
  const uint16_t* residual;   /* [M][H] BF16 added before rounding, or NULL */
  uint16_t* out;              /* [M][H] BF16 */
  void* workspace;            /* device scratch, >= moe_nvfp4_workspace_bytes(...) */
  int64_t workspace_bytes;
  int64_t M, E, k, H, I;
  int64_t dense_min_rows;     /* three-launch schedule: slots with at least this many rows
                                 use BF16 MFMA (above M = never; 0 = library default, by
                                 M: 16 for M <= 8, 3 for M <= 16, 6 for M <= 32, 8 above;
                                 16 in moe_nvfp4_route_decode) */
  int32_t schedule;           /* 0 = library choice, 2 = three launches,
                                 3 = two launches (per-row down + combine) */
  /* Optional, moe_nvfp4_route_decode only (NULL = none; moe_nvfp4_decode rejects
     it): a dense projection of the same rows, proj_out[M][proj_n] = bf16_rne(
     x W_p^T) as nvfp4_skinny_gemm computes it, bit for bit, with W_p packed
     G = 1, N = proj_n, K = H. Its blocks ride in the down launch, so the
     projection costs no launch of its own (for a layer chain that projects
     every layer's input, e.g. 2048 -> 64, beside the MoE block). Needs
     H = 2048, M <= 16, proj_n <= 4096, k (+1 with a shared expert) >= 4,
     proj_w and proj_out 16-byte aligned. Its blocks read x while other
     blocks of the same launch write out: out and proj_out must not overlap x
     (NVFP4MOE_ERR_BAD_SHAPE; residual == out stays fine, each output element
     is read and written by one thread). */
  const void* proj_w;
  int64_t proj_n;
  uint16_t* proj_out;
} moe_nvfp4_args;

/* Workspace bytes for moe_nvfp4_decode / moe_nvfp4_route_decode: h rows
 * [M*k (+M)][I] and expert outputs [M*k (+M)][H] as 32-bit words (the
 * two-launch schedule uses the h rows only). Every call writes what it reads
 * before reading it, so the workspace needs no initialisation and can be
 * reused (and replayed inside a HIP graph) as it is. A workspace serves one
 * call at a time: calls that may overlap (different streams) need their own. */
int64_t moe_nvfp4_workspace_bytes(int64_t M, int64_t E, int64_t k, int64_t H, int64_t I,
                                  int32_t has_shared);

/* out[m] = bf16_rne( sum_j w[m][j] * y_{ids[m][j]}(x[m]) + y_shared(x[m]) + residual[m] ),
 * y_e(x) = W_dn,e ( silu(u[0:I]) * u[I:2I] ),  u = W_gu,e x,  silu(a) = a / (1 + e^-a),
 * with FP32 accumulation and FP32 h. The slot sum runs in j order, then the
 * shared term, then the residual; the result is bit-reproducible from run to
 * run (no floating-point atomics).
 * Schedules: three launches (gate_up, down, combine) or two launches (gate_up,
 * then one block per (row, down tile) that runs the row's k pairs (+ the
 * shared expert) on that tile and sums them in place: no y round trip and no
 * combine launch, at the cost of reading a tile once per pair instead of once
 * per expert, which with few rows is nearly the same set). The library's choice (0) is two
 * launches for M <= 8 when M < dense_min_rows or the shape has no MFMA path,
 * else three; schedule 3 asks for two launches and returns
 * NVFP4MOE_ERR_UNSUPPORTED unless M < dense_min_rows or the shape has no
 * MFMA path (the per-row kernel needs FP32 h for every pair). In the
 * two- and three-launch schedules,
 * when H = 2048 and I = 512,
 * slots with at least dense_min_rows rows run on BF16 MFMA: weights exact in
 * BF16, x as stored, h as a hi + lo BF16 pair (relative error <= 2^-17).
 * Extra support-set conditions: H % 32 == 0 and I % 32 == 0 (each at most
 * 65536), and I is a multiple of the rows per tile of gate_up, 16384 / Kp with
 * Kp the largest 32 * 2^j <= 2048 dividing H (the up half then starts on a row
 * block: for H % 256 == 0, I % 64 == 0 is enough).
 * Returns NVFP4MOE_ERR_WORKSPACE if the workspace is too small and
 * NVFP4MOE_ERR_BAD_SHAPE for a schedule other than 0, 2 or 3. */
int32_t moe_nvfp4_decode(const moe_nvfp4_args* args, hipStream_t stream);

/* moe_route_topk (top-k and weights only, no grouping) and moe_nvfp4_decode
 * in one call of two launches, for few rows: the routing is done inside the
 * gate_up launch, one block per (pair, tile) selecting its row's experts with
 * the same per-row routine as moe_route_topk (so ids and w are bit-identical
 * to it), and the down launch sums each row's pairs in place (schedule 3 of
 * moe_nvfp4_decode). logits [M][E] FP32 and bias [E] FP32 (or NULL) as in
 * moe_route_topk. In args, ids [M][k] and w [M][k] are OUTPUTS (written with
 * the routing; the const of the struct fields is cast away), the grouping
 * arrays (offsets, pairs, active, active_offsets, n_active) and schedule are
 * not used; everything else is as for moe_nvfp4_decode, the output
 * bit-identical to moe_route_topk + moe_nvfp4_decode with schedule 3.
 * Reading a weight tile per pair rather than per expert suits small M (up to
 * about 8; without a shared expert and with routing spread evenly over the
 * experts it stays ahead of grouping at least to M = 24, with skewed routing
 * or a shared expert grouping wins from about M = 12); NVFP4MOE_ERR_UNSUPPORTED
 * when H = 2048, I = 512 and M >= dense_min_rows (pass a larger value beyond
 * M = 15: this path never uses the MFMA products). The workspace holds the h rows only: (M*k (+M)) * I * 4
 * bytes rounded up to 256 suffice (moe_nvfp4_workspace_bytes is more). */
int32_t moe_nvfp4_route_decode(const moe_nvfp4_args* args, const float* logits, const float* bias,
                               hipStream_t stream);

/* moe_nvfp4_route_decode for callers that cannot allocate device memory (code
 * under HIP graph capture that must not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the same launches, with the h rows in a
 * scratch array of the library instead of args->workspace (workspace and
 * workspace_bytes are ignored and may be NULL / 0). The array is a static
 * device array of 4 MiB (4194304 bytes); each GPU the library runs on holds
 * its own copy until the process ends, and the call allocates nothing. The
 * h rows take (M*k (+M with a shared expert)) * I * 4 bytes rounded up to
 * 256; a call that needs more returns NVFP4MOE_ERR_UNSUPPORTED before
 * launching. The first call on a device looks up that device's copy (the
 * current device's: call with the stream's device current). Every call on a
 * GPU shares that GPU's one array, which keeps the last call's contents (each
 * call writes the rows it reads first, so nothing needs clearing): calls that
 * may overlap on one GPU (different streams, different host threads) race and
 * must be ordered by the caller. Everything else, outputs included, is as for
 * moe_nvfp4_route_decode, bit for bit. */
int32_t moe_nvfp4_route_decode_static(const moe_nvfp4_args* args, const float* logits,
                                      const float* bias, hipStream_t stream);

/* ---- read ceiling (measurement) ---------------------------------------------------------
 *
 * The pages judge a decode step by the memory bandwidth it reaches against
 * the card's ([Weakest] page, "One config is the weakest card's config": the
 * decode roofline as bandwidth over the weight bytes read). This reads a buffer
 * once with the 16-byte nontemporal loads the weight streams use and nothing
 * else, so its rate is the ceiling those streams can reach on this chip, to
 * set beside the 8 TB/s peak.
 * nvfp4moe_stream_blocks(bytes): the number of workgroups (and sink words)
 * used for `bytes`, at most 8192; NVFP4MOE_ERR_BAD_SHAPE for bytes < 16.
 * nvfp4moe_stream_read: src (device, 16-byte aligned, bytes % 16 == 0,
 * bytes >= 16) is read once; workgroup b writes to sink[b] (device) the XOR
 * of the 32-bit words it read, so the XOR of the sink words is the XOR of the
 * whole buffer. sink_words below nvfp4moe_stream_blocks(bytes) gives
 * NVFP4MOE_ERR_WORKSPACE. */
int64_t nvfp4moe_stream_blocks(int64_t bytes);
int32_t nvfp4moe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
