/*
 * synth.h - seeded, counter-based generator of synthetic inputs.
 *
 * This module only produces input bytes: uniform E2M1 code bytes, log-uniform
 * E4M3 scale codes, BF16 / FP32 normal samples and Zipf+Gumbel router logits.
 * It holds none of the arithmetic of the NVFP4 MoE contraction (no decoding,
 * no products, no routing), and both the float64 oracle and the GPU library
 * consume its output unchanged.
 *
 * Every value is a pure function of (key, index): element i of a stream keyed
 * by `key` is SplitMix64 evaluated at counter i+1 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014), so any
 * sub-range can be produced on its own and fills parallelise without changing
 * the result.
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* SplitMix64 output mixer (the finaliser of the published generator). */
uint64_t synth_mix(uint64_t z);
/* Derives a stream key from a seed and four coordinates (config, layer,
 * tensor, expert). */
uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d);
/* Element i of stream `key`: the (i+1)-th SplitMix64 output from state `key`. */
uint64_t synth_u64(uint64_t key, uint64_t i);

/* Uniform random bytes. As packed E2M1 code pairs this draws every one of the
 * 16 codes, including -0, with equal probability. nthreads <= 0: automatic. */
void synth_fill_bytes(uint64_t key, uint8_t* out, int64_t n, int nthreads);

/* E4M3 scale codes, log-uniform: u ~ U[lo_log2, hi_log2), value 2^u rounded
 * to the nearest E4M3 value (ties never occur on the 53-bit grid). Only
 * positive normal codes result; requires -6 <= lo_log2 < hi_log2 <= 8. */
int synth_fill_scales(uint64_t key, uint8_t* out, int64_t n, double lo_log2,
                      double hi_log2, int nthreads);

/* Normal samples N(mean, std^2) via Box-Muller in double, rounded to FP32. */
void synth_fill_normal_f32(uint64_t key, float* out, int64_t n, double mean, double std);

/* Normal samples rounded first to FP32, then to BF16 with round-to-nearest-
 * even. Returned as raw BF16 bit patterns. */
void synth_fill_normal_bf16(uint64_t key, uint16_t* out, int64_t n, double mean, double std);

/* Router logits with Zipf expert popularity: logit[m][e] = ln p(rank(e)) +
 * Gumbel(0,1), p(r) proportional to r^-s for ranks r = 1..E, rank = a seeded
 * permutation of the experts (Fisher-Yates on stream perm_key). The top-k of
 * each row is then a weighted sample without replacement (Gumbel-top-k). */
void synth_fill_zipf_gumbel(uint64_t key, uint64_t perm_key, float* out, int64_t M,
                            int64_t E, double s);

/* The same fills for G streams at once: matrix g of `per` bytes uses keys[g].
 * Threads split the matrices. */
void synth_fill_bytes_keys(const uint64_t* keys, int64_t G, uint8_t* out, int64_t per,
                           int nthreads);
int synth_fill_scales_keys(const uint64_t* keys, int64_t G, uint8_t* out, int64_t per,
                           double lo_log2, double hi_log2, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
