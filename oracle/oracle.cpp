/*
 * oracle.cpp - float64 reference for the NVFP4 MoE decode path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library. Every step is its
 * plain definition evaluated in double, in the order the definition states.
 * See oracle.h for the layouts and for what each function follows.
 */
#include "oracle.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

/* ---- threads ------------------------------------------------------------------
 * The products and the MoE block split their outputs into independent jobs
 * (rows of W, or an expert's (row, slot) pairs) over a few threads. A job
 * writes only its own outputs and computes every one of them exactly as the
 * single-threaded loop does, so the result is bit-identical for any count. */
static std::atomic<int> g_threads{1};

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int oracle_threads(void) { return g_threads; }

/* Threads that parallel_jobs uses for njobs jobs. */
static int64_t job_workers(int64_t njobs) {
  return std::max<int64_t>(1, std::min<int64_t>(g_threads, njobs));
}

/* fn(job, worker) for job in [0, njobs), jobs handed out one at a time to
 * job_workers(njobs) threads; worker in [0, job_workers(njobs)) names the
 * thread, for state a thread keeps between its jobs. */
template <class F>
static void parallel_jobs(int64_t njobs, F fn) {
  const int64_t nt = job_workers(njobs);
  if (nt <= 1) {
    for (int64_t j = 0; j < njobs; ++j) fn(j, 0);
    return;
  }
  std::atomic<int64_t> next{0};
  auto worker = [&](int64_t t) {
    for (int64_t j = next++; j < njobs; j = next++) fn(j, t);
  };
  std::vector<std::thread> pool;
  for (int64_t t = 1; t < nt; ++t) pool.emplace_back(worker, t);
  worker(0);
  for (auto& th : pool) th.join();
}

/* ---- NVFP4 element and scale decoding ------------------------------------- */

/* E2M1 (OCP MX FP4): bit 3 sign, bits 2..1 exponent with bias 1, bit 0
 * mantissa. Exponent field 0 is subnormal: 0.5 * m. Otherwise
 * (1 + m/2) * 2^(e-1). The values are 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 * negatives (code 8 is -0). */
double oracle_e2m1(uint32_t code) {
  code &= 15u;
  const int sign = (code >> 3) & 1;
  const int e = (code >> 1) & 3;
  const int m = code & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * m;
  else
    mag = (1.0 + 0.5 * m) * std::ldexp(1.0, e - 1);
  return sign ? -mag : mag;
}

/* E4M3 (OCP 8-bit floating point, the "FN" variant used for NVFP4 block
 * scales): bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa.
 * Exponent 15 with mantissa 7 is NaN (no infinities). Exponent 0 is
 * subnormal: (m/8) * 2^-6. Otherwise (1 + m/8) * 2^(e-7). */
double oracle_e4m3(uint32_t byte) {
  byte &= 255u;
  const int sign = (byte >> 7) & 1;
  const int e = (byte >> 3) & 15;
  const int m = byte & 7;
  double mag;
  if (e == 15 && m == 7)
    mag = std::numeric_limits<double>::quiet_NaN();
  else if (e == 0)
    mag = (m / 8.0) * std::ldexp(1.0, -6);
  else
    mag = (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
  return sign ? -mag : mag;
}

/* BF16 is the upper half of an IEEE binary32. */
double oracle_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

/* Element (n, k) of matrix g in the canonical layout. */
static inline uint32_t code_at(const uint8_t* codes, int64_t N, int64_t K, int64_t gi, int64_t n,
                               int64_t k) {
  const uint8_t b = codes[(gi * N + n) * (K / 2) + k / 2];
  return (k & 1) ? (b >> 4) : (b & 15u);
}

static inline uint32_t scale_at(const uint8_t* scales, int64_t N, int64_t K, int64_t gi,
                                int64_t n, int64_t k) {
  return scales[(gi * N + n) * (K / 16) + k / 16];
}

/* Row n of matrix gi: W[n][k] = e2m1(code) * e4m3(scale of the 16-block
 * holding k) * g, for k = 0 .. K-1. */
static void dequant_row(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t N,
                        int64_t K, int64_t gi, int64_t n, double* row) {
  for (int64_t k = 0; k < K; ++k)
    row[k] = oracle_e2m1(code_at(codes, N, K, gi, n, k)) *
             oracle_e4m3(scale_at(scales, N, K, gi, n, k)) * (double)g[gi];
}

void oracle_dequant(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t G,
                    int64_t N, int64_t K, double* out) {
  for (int64_t gi = 0; gi < G; ++gi)
    for (int64_t n = 0; n < N; ++n) dequant_row(codes, scales, g, N, K, gi, n, &out[(gi * N + n) * K]);
}

void oracle_dequant_f32(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t G,
                        int64_t N, int64_t K, float* out) {
  for (int64_t gi = 0; gi < G; ++gi)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const float vs = (float)(oracle_e2m1(code_at(codes, N, K, gi, n, k)) *
                                 oracle_e4m3(scale_at(scales, N, K, gi, n, k)));
        out[(gi * N + n) * K + k] = vs * g[gi];
      }
}

/* ---- skinny product --------------------------------------------------------- */

/* Rows of W per job in the threaded products. */
static const int64_t kRowsPerJob = 64;

/* y[m][n] = sum over k ascending of x[m][k] * W[n][k], in double. A job takes
 * kRowsPerJob rows of W: each row is decoded once, then multiplied with every
 * row of x. */
void oracle_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* codes,
                 const uint8_t* scales, float g, int64_t N, double* y) {
  std::vector<double> xd((size_t)(M * K));
  for (int64_t i = 0; i < M * K; ++i) xd[(size_t)i] = oracle_bf16(x[i]);
  parallel_jobs((N + kRowsPerJob - 1) / kRowsPerJob, [&](int64_t job, int64_t) {
    std::vector<double> W((size_t)K);
    for (int64_t n = job * kRowsPerJob; n < std::min(N, (job + 1) * kRowsPerJob); ++n) {
      dequant_row(codes, scales, &g, N, K, 0, n, W.data());
      for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += xd[(size_t)(m * K + k)] * W[(size_t)k];
        y[m * N + n] = acc;
      }
    }
  });
}

/* y[m][n] = (sum_k x[m][k] * e4m3(w[n][k])) * s, float64: the FP8 skinny product
 * with one scale per tensor (Elsa page, "An FP8 fast path"). */
void oracle_gemm_fp8(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w, double s,
                     int64_t N, double* y) {
  parallel_jobs((N + kRowsPerJob - 1) / kRowsPerJob, [&](int64_t job, int64_t) {
    for (int64_t n = job * kRowsPerJob; n < std::min(N, (job + 1) * kRowsPerJob); ++n)
      for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
          acc += oracle_bf16(x[m * K + k]) * oracle_e4m3(w[n * K + k]);
        y[m * N + n] = acc * s;
      }
  });
}

/* logits[m][e] = sum_h x[m][h] * w_r[e][h] in float64: the router projection in
 * front of top-k routing of the mixture-of-experts model (Elsa page, "The card
 * and the model"). x and w_r are BF16 bit patterns; w_r is [E][H]. */
void oracle_router_logits(const uint16_t* x, int64_t M, int64_t H, const uint16_t* w_r, int64_t E,
                          double* logits) {
  parallel_jobs(M, [&](int64_t m, int64_t) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += oracle_bf16(x[m * H + h]) * oracle_bf16(w_r[e * H + h]);
      logits[m * E + e] = acc;
    }
  });
}

/* ---- quantization: BF16 -> canonical NVFP4 ----------------------------------------
 * The pages say only that a BF16 head was turned into NVFP4 with NVIDIA's
 * model optimizer (the Qwen3.8-27B NVFP4 lm_head recipe page, "Files": its
 * lm_head quantization script) and
 * give no recipe. The reading used here is the plain amax one, every division
 * and product in FP32 (the precision the GPU kernel decides in):
 *   g   = fl32(amax / 2688) over the whole matrix (2688 = 6 * 448: the largest
 *         E2M1 magnitude times the largest E4M3 value), 1 if amax = 0;
 *   s_b = E4M3 nearest to fl32(amax_b / fl32(6 g)), ties to the even code,
 *         448 above 448 (amax_b over the 16 elements of block b along K);
 *   q   = sign of x, magnitude the E2M1 nearest to fl32(|x| / fl32(s_b g)),
 *         ties to the even code, 6 above 6; magnitude 0 when s_b g = 0.
 * The nearest-value searches below scan the value tables directly. */

/* Nearest non-negative finite E4M3 code to t >= 0, ties to the even code. */
uint32_t oracle_e4m3_rne(float t) {
  if (t >= 448.0f) return 0x7Eu;  // saturate (a distance search loses ties far out)
  uint32_t best = 0;
  double bd = std::numeric_limits<double>::infinity();
  for (uint32_t c = 0; c <= 0x7E; ++c) {
    const double d = std::fabs(oracle_e4m3(c) - (double)t);
    if (d < bd || (d == bd && (c & 1u) == 0)) {
      best = c;
      bd = d;
    }
  }
  return best;
}

/* Nearest E2M1 magnitude code (0..7) to v >= 0, ties to the even code. */
uint32_t oracle_e2m1_rne(float v) {
  if (v >= 6.0f) return 7u;  // saturate
  uint32_t best = 0;
  double bd = std::numeric_limits<double>::infinity();
  for (uint32_t c = 0; c < 8; ++c) {
    const double d = std::fabs(oracle_e2m1(c) - (double)v);
    if (d < bd || (d == bd && (c & 1u) == 0)) {
      best = c;
      bd = d;
    }
  }
  return best;
}

static inline float bf16_f32(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

void oracle_quantize_nvfp4(const uint16_t* x, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* scales, float* g) {
  for (int64_t gi = 0; gi < G; ++gi) {
    const uint16_t* xm = x + gi * N * K;
    float amax = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) amax = std::max(amax, std::fabs(bf16_f32(xm[i])));
    const float gv = amax > 0.0f ? amax / 2688.0f : 1.0f;
    g[gi] = gv;
    const float six_g = 6.0f * gv;
    for (int64_t n = 0; n < N; ++n)
      for (int64_t b = 0; b < K / 16; ++b) {
        const uint16_t* xb = xm + n * K + b * 16;
        float amax_b = 0.0f;
        for (int i = 0; i < 16; ++i) amax_b = std::max(amax_b, std::fabs(bf16_f32(xb[i])));
        const uint32_t sc = oracle_e4m3_rne(amax_b / six_g);
        scales[(gi * N + n) * (K / 16) + b] = (uint8_t)sc;
        const float sg = (float)oracle_e4m3(sc) * gv;
        for (int i = 0; i < 16; ++i) {
          const float v = bf16_f32(xb[i]);
          const uint32_t mag = sg > 0.0f ? oracle_e2m1_rne(std::fabs(v) / sg) : 0u;
          const uint32_t q = (std::signbit(v) ? 8u : 0u) | mag;
          uint8_t& byte = codes[(gi * N + n) * (K / 2) + (b * 16 + i) / 2];
          if (i % 2 == 0)
            byte = (uint8_t)q;
          else
            byte = (uint8_t)(byte | (q << 4));
        }
      }
  }
}

/* ---- routing ----------------------------------------------------------------- */

/* Does expert a come before expert b? Larger l' first, NaN after everything,
 * equal values (including +0 / -0, and two NaNs) by lower index. */
static bool route_before(const std::vector<float>& lp, int a, int b) {
  const float la = lp[(size_t)a], lb = lp[(size_t)b];
  const bool na = std::isnan(la), nb = std::isnan(lb);
  if (na != nb) return nb;
  if (!na && la != lb) return la > lb;
  return a < b;
}

int oracle_route_topk(const float* logits, const float* bias, int64_t M, int64_t E, int64_t k,
                      int32_t* ids, double* w) {
  if (k < 1 || k > E) return -1;
  std::vector<float> lp((size_t)E);
  std::vector<int> order((size_t)E);
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t e = 0; e < E; ++e) {
      const float l = logits[m * E + e];
      lp[(size_t)e] = bias ? (float)(l + bias[e]) : l; /* one FP32 add */
    }
    for (int64_t e = 0; e < E; ++e) order[(size_t)e] = (int)e;
    std::sort(order.begin(), order.end(), [&](int a, int b) { return route_before(lp, a, b); });
    for (int64_t j = 0; j < k; ++j) ids[m * k + j] = order[(size_t)j];
    /* softmax restricted to the selected experts, renormalised to sum 1 */
    const double top = (double)lp[(size_t)order[0]];
    double z = 0.0;
    for (int64_t j = 0; j < k; ++j) z += std::exp((double)lp[(size_t)order[(size_t)j]] - top);
    for (int64_t j = 0; j < k; ++j)
      w[m * k + j] = std::exp((double)lp[(size_t)order[(size_t)j]] - top) / z;
  }
  return 0;
}

void oracle_group_by_expert(const int32_t* ids, int64_t M, int64_t E, int64_t k, int32_t* counts,
                            int32_t* offsets, int32_t* pairs, int32_t* active,
                            int32_t* active_offsets, int32_t* n_active) {
  const int64_t P = M * k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t pos = 0;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t p = 0; p < P; ++p)
      if (ids[p] == e) pairs[pos++] = (int32_t)p;
  int32_t na = 0;
  for (int64_t e = 0; e < E; ++e)
    if (counts[e] > 0) active[na++] = (int32_t)e;
  for (int64_t s = na; s < E; ++s) active[s] = -1;
  for (int64_t s = 0; s <= E; ++s) active_offsets[s] = s < na ? offsets[active[s]] : (int32_t)P;
  *n_active = na;
}

/* ---- expert feed-forward -------------------------------------------------------- */

static double silu(double a) { return a / (1.0 + std::exp(-a)); }

/* u = W_gu x (2I outputs); h[i] = silu(u[i]) * u[I + i]; y = W_dn h. Gate is
 * rows 0..I-1 of the fused gate_up matrix, up is rows I..2I-1. */
static void ffn_dequantized(const double* x, int64_t H, int64_t I, const double* Wgu,
                            const double* Wdn, double* y) {
  std::vector<double> u((size_t)(2 * I)), h((size_t)I);
  for (int64_t n = 0; n < 2 * I; ++n) {
    double acc = 0.0;
    for (int64_t kk = 0; kk < H; ++kk) acc += x[kk] * Wgu[(size_t)(n * H + kk)];
    u[(size_t)n] = acc;
  }
  for (int64_t i = 0; i < I; ++i) h[(size_t)i] = silu(u[(size_t)i]) * u[(size_t)(I + i)];
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += h[(size_t)i] * Wdn[(size_t)(n * I + i)];
    y[n] = acc;
  }
}

void oracle_expert_ffn(const uint16_t* x, int64_t H, int64_t I, const uint8_t* gu_codes,
                       const uint8_t* gu_scales, float gu_g, const uint8_t* dn_codes,
                       const uint8_t* dn_scales, float dn_g, double* y) {
  std::vector<double> Wgu((size_t)(2 * I * H)), Wdn((size_t)(H * I)), xd((size_t)H);
  oracle_dequant(gu_codes, gu_scales, &gu_g, 1, 2 * I, H, Wgu.data());
  oracle_dequant(dn_codes, dn_scales, &dn_g, 1, H, I, Wdn.data());
  for (int64_t kk = 0; kk < H; ++kk) xd[(size_t)kk] = oracle_bf16(x[kk]);
  ffn_dequantized(xd.data(), H, I, Wgu.data(), Wdn.data(), y);
}

/* ---- MoE block ------------------------------------------------------------------- */

/* The (row, slot) pairs of one expert, or shared-expert rows, per job. */
static const int64_t kPairsPerJob = 8;

struct FfnJob {
  int64_t e;      /* expert (-1: the shared expert) */
  int64_t first;  /* index into the expert's pair list (or the first row) */
  int64_t count;
};

void oracle_moe_block_f64(const double* x, int64_t M, int64_t H, int64_t I, int64_t E, int64_t k,
                          const int32_t* ids, const double* w, const uint8_t* gu_codes,
                          const uint8_t* gu_scales, const float* gu_g, const uint8_t* dn_codes,
                          const uint8_t* dn_scales, const float* dn_g, const uint8_t* sgu_codes,
                          const uint8_t* sgu_scales, const float* sgu_g, const uint8_t* sdn_codes,
                          const uint8_t* sdn_scales, const float* sdn_g, const double* residual,
                          double* out) {
  const int64_t P = M * k;
  /* y_p for every (row, slot) pair p = m*k + j, through expert ids[p], and
   * the shared expert's output for every row. Each job dequantizes its expert
   * (a thread keeps the last one it decoded) and applies it to its pairs. */
  std::vector<std::vector<int64_t>> pairs_of((size_t)E);
  for (int64_t p = 0; p < P; ++p) pairs_of[(size_t)ids[p]].push_back(p);
  std::vector<FfnJob> jobs;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t f = 0; f < (int64_t)pairs_of[(size_t)e].size(); f += kPairsPerJob)
      jobs.push_back({e, f, std::min<int64_t>(kPairsPerJob, (int64_t)pairs_of[(size_t)e].size() - f)});
  if (sgu_codes)
    for (int64_t r = 0; r < M; r += kPairsPerJob)
      jobs.push_back({-1, r, std::min<int64_t>(kPairsPerJob, M - r)});
  std::vector<double> Y((size_t)(P * H)), S(sgu_codes ? (size_t)(M * H) : 0);
  struct Held {  /* a thread's decoded expert, kept between its jobs */
    std::vector<double> Wgu, Wdn;
    int64_t e = -2;
  };
  std::vector<Held> held((size_t)job_workers((int64_t)jobs.size()));
  parallel_jobs((int64_t)jobs.size(), [&](int64_t jn, int64_t worker) {
    const FfnJob& J = jobs[(size_t)jn];
    std::vector<double>& Wgu = held[(size_t)worker].Wgu;
    std::vector<double>& Wdn = held[(size_t)worker].Wdn;
    if (held[(size_t)worker].e != J.e) {
      Wgu.resize((size_t)(2 * I * H));
      Wdn.resize((size_t)(H * I));
      if (J.e < 0) {
        oracle_dequant(sgu_codes, sgu_scales, sgu_g, 1, 2 * I, H, Wgu.data());
        oracle_dequant(sdn_codes, sdn_scales, sdn_g, 1, H, I, Wdn.data());
      } else {
        oracle_dequant(gu_codes + J.e * (2 * I * H / 2), gu_scales + J.e * (2 * I * H / 16),
                       gu_g + J.e, 1, 2 * I, H, Wgu.data());
        oracle_dequant(dn_codes + J.e * (H * I / 2), dn_scales + J.e * (H * I / 16), dn_g + J.e,
                       1, H, I, Wdn.data());
      }
      held[(size_t)worker].e = J.e;
    }
    for (int64_t q = J.first; q < J.first + J.count; ++q) {
      if (J.e < 0) {
        ffn_dequantized(&x[q * H], H, I, Wgu.data(), Wdn.data(), &S[(size_t)(q * H)]);
      } else {
        const int64_t p = pairs_of[(size_t)J.e][(size_t)q];
        ffn_dequantized(&x[(p / k) * H], H, I, Wgu.data(), Wdn.data(), &Y[(size_t)(p * H)]);
      }
    }
  });
  /* combine: routing-weighted sum over the k slots in slot order, then the
   * shared expert with weight 1, then the residual */
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j)
        acc += w[m * k + j] * Y[(size_t)((m * k + j) * H + n)];
      if (sgu_codes) acc += S[(size_t)(m * H + n)];
      if (residual) acc += residual[m * H + n];
      out[m * H + n] = acc;
    }
}

void oracle_moe_block(const uint16_t* x, int64_t M, int64_t H, int64_t I, int64_t E, int64_t k,
                      const int32_t* ids, const double* w, const uint8_t* gu_codes,
                      const uint8_t* gu_scales, const float* gu_g, const uint8_t* dn_codes,
                      const uint8_t* dn_scales, const float* dn_g, const uint8_t* sgu_codes,
                      const uint8_t* sgu_scales, const float* sgu_g, const uint8_t* sdn_codes,
                      const uint8_t* sdn_scales, const float* sdn_g, const uint16_t* residual,
                      double* out) {
  /* BF16 -> double is exact, so this is the float64 block on the same values */
  std::vector<double> xd((size_t)(M * H)), rd(residual ? (size_t)(M * H) : 0);
  for (int64_t i = 0; i < M * H; ++i) xd[(size_t)i] = oracle_bf16(x[i]);
  if (residual)
    for (int64_t i = 0; i < M * H; ++i) rd[(size_t)i] = oracle_bf16(residual[i]);
  oracle_moe_block_f64(xd.data(), M, H, I, E, k, ids, w, gu_codes, gu_scales, gu_g, dn_codes,
                       dn_scales, dn_g, sgu_codes, sgu_scales, sgu_g, sdn_codes, sdn_scales, sdn_g,
                       residual ? rd.data() : nullptr, out);
}

int oracle_moe_decode(const uint16_t* x, const float* logits, const float* bias, int64_t M,
                      int64_t H, int64_t I, int64_t E, int64_t k, const uint8_t* gu_codes,
                      const uint8_t* gu_scales, const float* gu_g, const uint8_t* dn_codes,
                      const uint8_t* dn_scales, const float* dn_g, const uint8_t* sgu_codes,
                      const uint8_t* sgu_scales, const float* sgu_g, const uint8_t* sdn_codes,
                      const uint8_t* sdn_scales, const float* sdn_g, const uint16_t* residual,
                      int32_t* ids, double* w, double* out) {
  if (oracle_route_topk(logits, bias, M, E, k, ids, w) != 0) return -1;
  oracle_moe_block(x, M, H, I, E, k, ids, w, gu_codes, gu_scales, gu_g, dn_codes, dn_scales,
                   dn_g, sgu_codes, sgu_scales, sgu_g, sdn_codes, sdn_scales, sdn_g, residual,
                   out);
  return 0;
}
