// abi_main.cpp - the C ABI's host-side validation under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py): every call below is
// rejected before any launch, so no GPU is needed; the sanitizers check the
// validation code itself (argument reads, overflow in the size arithmetic,
// the error-detail formatting).
#include <cstdio>
#include <cstring>

#include "nvfp4moe.h"

#define EXPECT(call, code)                                                        \
  do {                                                                            \
    const long long got = (long long)(call);                                      \
    if (got != (code)) {                                                          \
      std::printf("FAIL %s: %lld (%s)\n", #call, got, nvfp4moe_last_error_detail()); \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main() {
  void* f = reinterpret_cast<void*>(4096);
  auto u8 = static_cast<uint8_t*>(f);
  auto u16 = static_cast<uint16_t*>(f);
  auto f32 = static_cast<float*>(f);
  auto i32 = static_cast<int32_t*>(f);
  EXPECT(nvfp4_packed_bytes(1, 8, 96), 2 * 0 + 3 * 9216 + 256);
  EXPECT(nvfp4_packed_bytes(1, 8, 48), NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(nvfp4_packed_bytes(0, 8, 64), NVFP4MOE_ERR_BAD_SHAPE);
  EXPECT(nvfp4_packed_bytes(1, (int64_t)1 << 62, 64), NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(nvfp4_pack(nullptr, u8, f32, 1, 8, 64, f, nullptr), NVFP4MOE_ERR_NULL_ARG);
  EXPECT(nvfp4_skinny_gemm(u16, 0, 64, f, 8, u16, nullptr), NVFP4MOE_ERR_BAD_SHAPE);
  EXPECT(nvfp4_skinny_gemm(u16, 1, 4100, f, 8, u16, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(nvfp4_skinny_gemm(u16, 1, 64, f, (int64_t)1 << 62, u16, nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(fp8_skinny_gemm(u16, 1, 512, u8, f32, 8, u16, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(nvfp4_quantize(u16, 1, 8, 40, u8, u8, f32, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route_topk(f32, nullptr, 4, 257, 8, i32, f32, i32, i32, i32, i32, i32, i32,
                        nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route_topk(f32, nullptr, (int64_t)1 << 40, 256, 8, i32, f32, i32, i32, i32, i32, i32,
                        i32, nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(moe_nvfp4_workspace_bytes(4, 256, 8, 2048, 512, 0), 4 * 8 * (512 + 2048) * 4);
  EXPECT(moe_nvfp4_workspace_bytes(4, 256, 8, 2048, 100, 0), NVFP4MOE_ERR_UNSUPPORTED);
  moe_nvfp4_args a;
  std::memset(&a, 0, sizeof(a));
  a.x = u16;
  a.ids = i32;
  a.w = f32;
  a.offsets = a.pairs = a.active = a.active_offsets = a.n_active = i32;
  a.w_gate_up = a.w_down = f;
  a.out = u16;
  a.workspace = f;
  a.workspace_bytes = 1 << 30;
  a.M = 4; a.E = 256; a.k = 8; a.H = 2048; a.I = 512;
  EXPECT(moe_nvfp4_decode(nullptr, nullptr), NVFP4MOE_ERR_NULL_ARG);
  a.schedule = 1;
  EXPECT(moe_nvfp4_decode(&a, nullptr), NVFP4MOE_ERR_BAD_SHAPE);
  a.schedule = 0;
  a.M = (int64_t)1 << 40;
  EXPECT(moe_nvfp4_decode(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
  a.M = 4;
  a.H = 96; a.I = 256;
  EXPECT(moe_nvfp4_decode(&a, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
  a.H = 2048; a.I = 512;
  a.workspace_bytes = 16;
  EXPECT(moe_nvfp4_route_decode(&a, f32, nullptr, nullptr), NVFP4MOE_ERR_WORKSPACE);
  a.workspace_bytes = 1 << 30;
  a.proj_w = f; a.proj_n = 64; a.proj_out = u16;  // proj_out == x: overlap
  EXPECT(moe_nvfp4_route_decode(&a, f32, nullptr, nullptr), NVFP4MOE_ERR_BAD_SHAPE);
  a.proj_w = nullptr;
  a.M = 200; a.I = 1024; a.dense_min_rows = 1 << 20;
  EXPECT(moe_nvfp4_route_decode_static(&a, f32, nullptr, nullptr), NVFP4MOE_ERR_UNSUPPORTED);
  EXPECT(nvfp4moe_stream_read(f, 40, static_cast<uint32_t*>(f), 1, nullptr),
         NVFP4MOE_ERR_UNSUPPORTED);
  if (std::strcmp(nvfp4moe_strerror(-3), "NVFP4MOE_ERR_UNSUPPORTED") != 0) return 1;
  std::puts("abi sanitized run: ok");
  return 0;
}
