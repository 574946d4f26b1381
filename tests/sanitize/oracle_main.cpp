// oracle_main.cpp - runs every oracle entry point on small inputs, for a build
// with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py):
// any out-of-bounds access, leak or undefined operation ends the run with an error.
#include <cstdio>
#include <cstring>
#include <vector>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return (uint32_t)(g_state >> 16);
}

int main() {
  for (int threads : {1, 3}) {
    oracle_set_threads(threads);
    const int64_t M = 5, H = 96, I = 64, E = 6, k = 2;
    std::vector<uint16_t> x(M * H), res(M * H), wr(E * H);
    for (auto& v : x) v = (uint16_t)(0x3F00 + next_u32() % 256);  // BF16 in [0.5, 2)
    for (auto& v : res) v = (uint16_t)(0xBF00 + next_u32() % 256);
    for (auto& v : wr) v = (uint16_t)(0x3C00 + next_u32() % 256);
    std::vector<uint8_t> gu_c(E * 2 * I * H / 2), gu_s(E * 2 * I * H / 16);
    std::vector<uint8_t> dn_c(E * H * I / 2), dn_s(E * H * I / 16);
    for (auto& v : gu_c) v = (uint8_t)next_u32();
    for (auto& v : dn_c) v = (uint8_t)next_u32();
    for (auto& v : gu_s) v = (uint8_t)(0x18 + next_u32() % 0x40);
    for (auto& v : dn_s) v = (uint8_t)(0x18 + next_u32() % 0x40);
    std::vector<float> gu_g(E, 1.0f / 512), dn_g(E, 1.0f / 256), logits(M * E), bias(E);
    for (auto& v : logits) v = (float)(next_u32() % 1000) / 250.0f - 2.0f;
    for (auto& v : bias) v = (float)(next_u32() % 100) / 100.0f;
    std::vector<int32_t> ids(M * k);
    std::vector<double> w(M * k), out(M * H), y(M * H);
    if (oracle_moe_decode(x.data(), logits.data(), bias.data(), M, H, I, E, k, gu_c.data(),
                          gu_s.data(), gu_g.data(), dn_c.data(), dn_s.data(), dn_g.data(),
                          gu_c.data(), gu_s.data(), gu_g.data(), dn_c.data(), dn_s.data(),
                          dn_g.data(), res.data(), ids.data(), w.data(), out.data()) != 0)
      return 2;
    std::vector<int32_t> counts(E), offsets(E + 1), pairs(M * k), active(E), aoff(E + 1), na(1);
    oracle_group_by_expert(ids.data(), M, E, k, counts.data(), offsets.data(), pairs.data(),
                           active.data(), aoff.data(), na.data());
    std::vector<double> xd(M * H);
    for (int64_t i = 0; i < M * H; ++i) xd[i] = oracle_bf16(x[i]);
    oracle_moe_block_f64(xd.data(), M, H, I, E, k, ids.data(), w.data(), gu_c.data(),
                         gu_s.data(), gu_g.data(), dn_c.data(), dn_s.data(), dn_g.data(), nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, xd.data(), y.data());
    oracle_expert_ffn(x.data(), H, I, gu_c.data(), gu_s.data(), gu_g[0], dn_c.data(),
                      dn_s.data(), dn_g[0], y.data());
    std::vector<double> yg(M * 2 * I), lg(M * E);
    oracle_gemm(x.data(), M, H, gu_c.data(), gu_s.data(), 0.37f, 2 * I, yg.data());
    std::vector<uint8_t> w8(2 * I * H);
    for (auto& v : w8) v = (uint8_t)(next_u32() % 0x7F);
    oracle_gemm_fp8(x.data(), M, H, w8.data(), 0.5, 2 * I, yg.data());
    oracle_router_logits(x.data(), M, H, wr.data(), E, lg.data());
    std::vector<double> deq(2 * I * H);
    std::vector<float> deq32(2 * I * H);
    oracle_dequant(gu_c.data(), gu_s.data(), gu_g.data(), 1, 2 * I, H, deq.data());
    oracle_dequant_f32(gu_c.data(), gu_s.data(), gu_g.data(), 1, 2 * I, H, deq32.data());
    std::vector<uint8_t> qc(2 * I * H / 2), qs(2 * I * H / 16);
    std::vector<float> qg(1);
    std::vector<uint16_t> xb(2 * I * H);
    for (auto& v : xb) v = (uint16_t)(next_u32() & 0xFF7F);  // finite BF16 of any sign
    oracle_quantize_nvfp4(xb.data(), 1, 2 * I, H, qc.data(), qs.data(), qg.data());
    for (uint32_t c = 0; c < 256; ++c) (void)oracle_e4m3(c);
    (void)oracle_e4m3_rne(3.0f);
    (void)oracle_e2m1_rne(2.5f);
  }
  std::puts("oracle sanitized run: ok");
  return 0;
}
