// api.hip - the extern "C" entry points of libnvfp4moe.so (see include/nvfp4moe.h).
//
// Every call validates on the host, launches on the caller's stream and
// returns; nothing is allocated, synchronised or read back.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "nvfp4moe.h"

#include "fp8.hpp"
#include "fused.hpp"
#include "gemm.hpp"
#include "moe.hpp"
#include "staged.hpp"
#include "pack.hpp"
#include "quant.hpp"
#include "route.hpp"
#include "router.hpp"
#include "stream.hpp"

static_assert(nvfp4moe::kMaxTopK == nvfp4moe::kRouteMaxK, "combine unrolls to the routing bound on k");

using namespace nvfp4moe;

// Scratch of moe_nvfp4_route_decode_static: the h rows of one call. Every GPU
// the library runs on holds its own copy until the process ends; host code
// never uses this name as an address (it is a host-side stand-in), only the
// address hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchBytes = 4 << 20;
constexpr int kScratchMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local char g_detail[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_detail[0] = '\0';
  return NVFP4MOE_OK;
}

int32_t launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(NVFP4MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// K of a packed matrix: a multiple of 32 (whole chunks), at most kMaxK.
constexpr int64_t kMaxK = 65536;
bool valid_k(int64_t K) { return K >= 32 && K <= kMaxK && K % 32 == 0; }
// Bounds that keep every size product of a packed tensor inside int64_t.
constexpr int64_t kMaxG = (int64_t)1 << 20;
constexpr int64_t kMaxN = (int64_t)1 << 32;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Do the byte ranges [p, p + pn) and [q, q + qn) share a byte?
bool overlaps(const void* p, int64_t pn, const void* q, int64_t qn) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qn && b < a + (uintptr_t)pn;
}

int grid_for(int64_t items, int64_t per_block, int64_t cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

template <template <int> class Launcher, typename... Args>
int32_t dispatch_l(int64_t L, Args&&... args) {
  switch (L) {
    case 1: return Launcher<1>::run(args...);
    case 2: return Launcher<2>::run(args...);
    case 4: return Launcher<4>::run(args...);
    case 8: return Launcher<8>::run(args...);
    case 16: return Launcher<16>::run(args...);
    case 32: return Launcher<32>::run(args...);
    case 64: return Launcher<64>::run(args...);
    default: return fail(NVFP4MOE_ERR_UNSUPPORTED, "K/32 = %lld", (long long)L);
  }
}

template <int L>
struct GemmLaunch {
  static int32_t run(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w, int64_t N,
                     uint16_t* y, hipStream_t s) {
    const int64_t blocks = row_blocks(N, K);  // one wave each
    const float* gp = reinterpret_cast<const float*>(w + gscale_offset(1, N, K));
    hipLaunchKernelGGL(skinny_gemm_kernel<L>, dim3(grid_for(blocks, 4, 1 << 30)), dim3(256), 0,
                       s, x, M, K, w, N, y, blocks, K / (L * 32), gp);
    return launched("nvfp4_skinny_gemm");
  }
};

// token_down_combine blocks: one wave per slot up to eight slots; eight waves
// for eight routed slots and the shared expert, wave 0 taking two (k <= 8, so
// nine slots means k = 8 with a shared expert).
template <int LI>
void launch_token_down(const MoeParams& p, hipStream_t s) {
  const int n = p.k + p.has_shared;
  const int grid = p.M * p.PD + p.proj_blocks;  // the projection's blocks first
  if (n <= 8)
    hipLaunchKernelGGL((token_down_combine_kernel<LI, false>), dim3(grid), dim3(n * 64), 0, s,
                       p);
  else
    hipLaunchKernelGGL((token_down_combine_kernel<LI, true>), dim3(grid), dim3((n - 1) * 64), 0,
                       s, p);
}

// One thread per output. Up to 65,536 outputs (M <= 32 at H = 2048) in blocks
// of one wave, which spreads them over every CU (M = 16: 44.93 -> 44.81 us;
// at M = 256, 256-thread blocks measured as fast as 64 or 128).
void launch_combine(const MoeParams& p, hipStream_t s) {
  const int64_t outs = (int64_t)p.M * p.H;
  if (outs <= 65536)
    hipLaunchKernelGGL(staged_combine_kernel<64>, dim3((unsigned)((outs + 63) / 64)), dim3(64), 0,
                       s, p);
  else
    hipLaunchKernelGGL(staged_combine_kernel<256>, dim3((unsigned)((outs + 255) / 256)), dim3(256),
                       0, s, p);
}

template <int LH, int LI, int RG, int RD, bool DENSE>
int32_t launch_staged(const MoeParams& p, hipStream_t s) {
  // many rows: the items take the slots heaviest first
  hipLaunchKernelGGL((staged_gate_kernel<LH, RG, DENSE, true>), dim3(p.slots * p.PG), dim3(64), 0,
                     s, p);
  hipLaunchKernelGGL((staged_down_kernel<LI, RD, DENSE, true>), dim3(p.slots * p.PD), dim3(64), 0,
                     s, p);
  launch_combine(p, s);
  return launched("moe_nvfp4_decode");
}

// One row per batch: gate_up with two waves per item (gate tile, up tile).
template <int LH, int LI, bool DENSE>
int32_t launch_staged_split(const MoeParams& p, bool token_major, hipStream_t s) {
  hipLaunchKernelGGL((staged_gate_split_kernel<LH, DENSE>), dim3(p.slots * p.PG), dim3(128), 0, s,
                     p);
  if (token_major) {
    launch_token_down<LI>(p, s);
    return launched("moe_nvfp4_decode");
  }
  // down: two rows per VALU batch where the shape is specialised (M = 16:
  // 46.8 -> 46.5 us; the generic kernel would spill at two)
  hipLaunchKernelGGL((staged_down_kernel<LI, (LI != 0 ? 2 : 1), DENSE, false>),
                     dim3(p.slots * p.PD), dim3(64), 0, s, p);
  launch_combine(p, s);
  return launched("moe_nvfp4_decode");
}

// Rows per batch: gate_up 1, 2 or 4, down at most 2 (register budget); the
// shapes without MFMA take one row at a time.
int32_t launch_staged_rows(const MoeParams& p, bool specialised, int rmax, bool token_major,
                           hipStream_t s) {
  if (rmax == 1 || token_major)
    return specialised ? launch_staged_split<64, 16, true>(p, token_major, s)
                       : launch_staged_split<0, 0, false>(p, token_major, s);
  if (!specialised) return launch_staged<0, 0, 1, 1, false>(p, s);
  return rmax == 2 ? launch_staged<64, 16, 2, 2, true>(p, s)
                   : launch_staged<64, 16, 4, 2, true>(p, s);
}

struct WsLayout {
  int64_t hp_off, yp_off, total;
};

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

// h [P][I], then y [P][H], as 32-bit words, P = M*k (+ M with a shared
// expert); every call overwrites what it reads, so the contents never carry
// from one call to the next. The two-launch schedule uses h only.
WsLayout ws_layout(int64_t M, int64_t k, int64_t H, int64_t I, bool shared) {
  const int64_t P = M * k + (shared ? M : 0);
  WsLayout w;
  w.hp_off = 0;
  w.yp_off = align256(P * I * 4);
  w.total = w.yp_off + align256(P * H * 4);
  return w;
}


}  // namespace

namespace {

int32_t check_route(const float* logits, int64_t M, int64_t E, int64_t k, int32_t* ids, float* w,
                    int32_t* counts, int32_t* offsets, int32_t* pairs, int32_t* active,
                    int32_t* active_offsets, int32_t* n_active) {
  if (!logits || !ids || !w || !counts || !offsets || !pairs || !active || !active_offsets ||
      !n_active)
    return fail(NVFP4MOE_ERR_NULL_ARG, "routing: null");
  if (M < 1 || E < 1 || k < 1) return fail(NVFP4MOE_ERR_BAD_SHAPE, "M, E, k must be >= 1");
  if (E > kRouteMaxE) return fail(NVFP4MOE_ERR_UNSUPPORTED, "E = %lld > 256", (long long)E);
  if (k > kRouteMaxK || k > E)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "k = %lld: need k <= min(8, E)", (long long)k);
  if (M * k > kGroupMaxPairs)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "M * k = %lld > %d", (long long)(M * k),
                kGroupMaxPairs);
  return ok();
}

// Top-k selection and grouping of validated logits.
int32_t launch_route(const float* logits, const float* bias, int64_t M, int64_t E, int64_t k,
                     int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* pairs,
                     int32_t* active, int32_t* active_offsets, int32_t* n_active,
                     hipStream_t stream) {
  if (M <= kRouteSingleBlockRows) {
    hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(1024), 0, stream, logits, bias, (int)M,
                       (int)E, (int)k, ids, w, counts, offsets, pairs, active, active_offsets,
                       n_active);
    return launched("moe_route_topk");
  }
  hipLaunchKernelGGL(route_rows_kernel, dim3(grid_for(M, kRowWaves, 1 << 20)),
                     dim3(kRowWaves * 64), 0, stream, logits, bias, (int)M, (int)E, (int)k, ids,
                     w);
  const int32_t st = launched("moe_route_topk rows");
  if (st != NVFP4MOE_OK) return st;
  if (M <= kGroupMaskRows)
    hipLaunchKernelGGL(group_rows_kernel, dim3(1), dim3(1024), 0, stream, ids, (int)M, (int)E,
                       (int)k, counts, offsets, pairs, active, active_offsets, n_active);
  else
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), 0, stream, ids, (int)M, (int)E, (int)k,
                       counts, offsets, pairs, active, active_offsets, n_active);
  return launched("moe_route_topk group");
}

}  // namespace

namespace {

// Validates the arguments and fills p. routed: the routing arrays come from
// moe_route_topk (moe_nvfp4_decode: h and y in the workspace); otherwise only
// ids and w, which the call writes (moe_nvfp4_route_decode: h only). scratch:
// when not null, used in place of a->workspace (which is then ignored).
int32_t prepare_decode(const moe_nvfp4_args* a, bool routed, MoeParams& p,
                       void* scratch = nullptr, int64_t scratch_bytes = 0) {
  if (!a) return fail(NVFP4MOE_ERR_NULL_ARG, "moe_nvfp4_decode: args is null");
  void* const wsp = scratch ? scratch : a->workspace;
  const int64_t ws_bytes = scratch ? scratch_bytes : a->workspace_bytes;
  if (!a->x || !a->ids || !a->w || !a->w_gate_up || !a->w_down || !a->out || !wsp ||
      (routed && (!a->offsets || !a->pairs || !a->active || !a->active_offsets || !a->n_active)))
    return fail(NVFP4MOE_ERR_NULL_ARG, "moe_nvfp4_decode: a required pointer is null");
  if ((a->shared_gate_up == nullptr) != (a->shared_down == nullptr))
    return fail(NVFP4MOE_ERR_NULL_ARG, "shared_gate_up and shared_down go together");
  const int64_t M = a->M, E = a->E, k = a->k, H = a->H, I = a->I;
  if (M < 1 || E < 1 || k < 1 || H < 1 || I < 1)
    return fail(NVFP4MOE_ERR_BAD_SHAPE, "M, E, k, H, I must be >= 1");
  if (E > kRouteMaxE || k > kRouteMaxK || k > E)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "need E <= 256 and k <= min(8, E)");
  if (!valid_k(H) || !valid_k(I))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "H and I must be multiples of 32 in [32, %lld]",
                (long long)kMaxK);
  if (I % rows_per_tile(H) != 0)
    return fail(NVFP4MOE_ERR_UNSUPPORTED,
                "I = %lld must be a multiple of the gate_up rows per tile, %lld (the up half "
                "starts on a row block)",
                (long long)I, (long long)rows_per_tile(H));
  if (M * k + M > (int64_t)1 << 24) return fail(NVFP4MOE_ERR_UNSUPPORTED, "M too large");
  // every grid (items x row blocks per matrix) must stay below 2^31 blocks
  const int64_t pg = I / rows_per_tile(H), pd = row_blocks(H, I);
  if ((M * k + M) * (pg > pd ? pg : pd) + 4096 > ((int64_t)1 << 31) - 1)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "M too large for the grid");
  if (a->schedule != 0 && a->schedule != 2 && a->schedule != 3)
    return fail(NVFP4MOE_ERR_BAD_SHAPE, "schedule must be 0, 2 or 3 (got %d)", (int)a->schedule);
  const bool shared = a->shared_gate_up != nullptr;
  const WsLayout ws = ws_layout(M, k, H, I, shared);
  const int64_t need = routed ? ws.total : ws.yp_off;
  if (ws_bytes < need)
    return fail(NVFP4MOE_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes,
                (long long)need);
  if (!aligned(a->x, 16) || !aligned(a->w_gate_up, 16) || !aligned(a->w_down, 16) ||
      !aligned(wsp, 256) || (shared && (!aligned(a->shared_gate_up, 16) ||
                                                 !aligned(a->shared_down, 16))))
    return fail(NVFP4MOE_ERR_UNSUPPORTED,
                "x and weights need 16-byte, workspace 256-byte alignment");

  std::memset(&p, 0, sizeof(p));
  p.x = a->x;
  p.ids = a->ids;
  p.w = a->w;
  p.offsets = a->offsets;
  p.pairs = a->pairs;
  p.active = a->active;
  p.active_offsets = a->active_offsets;
  p.n_active = a->n_active;
  p.gu = (const uint8_t*)a->w_gate_up;
  p.dn = (const uint8_t*)a->w_down;
  p.sgu = (const uint8_t*)a->shared_gate_up;
  p.sdn = (const uint8_t*)a->shared_down;
  p.residual = a->residual;
  p.out = a->out;
  uint8_t* wsb = (uint8_t*)wsp;
  p.M = (int)M;
  p.E = (int)E;
  p.k = (int)k;
  p.H = (int)H;
  p.I = (int)I;
  p.KpH = (int)panel_k(H);
  p.KpI = (int)panel_k(I);
  p.LH = p.KpH / 32;
  p.LI = p.KpI / 32;
  p.QH = (int)panels(H);
  p.QI = (int)panels(I);
  p.RH = (int)rows_per_tile(H);
  p.RI = (int)rows_per_tile(I);
  p.routed_slots = (int)(E < M * k ? E : M * k);
  p.has_shared = shared ? 1 : 0;
  p.slots = p.routed_slots + p.has_shared;
  p.gu_mat_bytes = matrix_bytes(2 * I, H);
  p.dn_mat_bytes = matrix_bytes(H, I);
  p.gu_g = (const float*)(p.gu + gscale_offset(E, 2 * I, H));
  p.dn_g = (const float*)(p.dn + gscale_offset(E, H, I));
  if (shared) {
    p.sgu_g = (const float*)(p.sgu + gscale_offset(1, 2 * I, H));
    p.sdn_g = (const float*)(p.sdn + gscale_offset(1, H, I));
  }
  p.PG = (int)pg;
  p.PD = (int)pd;
  p.pair_regs = M * k <= 128 ? (int)((M * k + 63) / 64) : 0;
  p.hp = (float*)(wsb + ws.hp_off);
  p.yp = (float*)(wsb + ws.yp_off);
  p.dense_min_rows = a->dense_min_rows > 0
                         ? (int)(a->dense_min_rows < (int64_t)1 << 30 ? a->dense_min_rows : 1 << 30)
                         : dense_rows_default(M, routed);
  return ok();
}

}  // namespace

extern "C" {

const char* nvfp4moe_strerror(int32_t status) {
  switch (status) {
    case NVFP4MOE_OK: return "NVFP4MOE_OK";
    case NVFP4MOE_ERR_NULL_ARG: return "NVFP4MOE_ERR_NULL_ARG";
    case NVFP4MOE_ERR_BAD_SHAPE: return "NVFP4MOE_ERR_BAD_SHAPE";
    case NVFP4MOE_ERR_UNSUPPORTED: return "NVFP4MOE_ERR_UNSUPPORTED";
    case NVFP4MOE_ERR_WORKSPACE: return "NVFP4MOE_ERR_WORKSPACE";
    case NVFP4MOE_ERR_HIP: return "NVFP4MOE_ERR_HIP";
    default: return "NVFP4MOE_ERR_UNKNOWN";
  }
}

const char* nvfp4moe_last_error_detail(void) { return g_detail; }

const char* nvfp4moe_version(void) { return "nvfp4moe 0.1 gfx950"; }

int64_t nvfp4_packed_bytes(int64_t G, int64_t N, int64_t K) {
  if (G < 1 || N < 1) return fail(NVFP4MOE_ERR_BAD_SHAPE, "G and N must be >= 1");
  if (G > kMaxG || N > kMaxN)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "G <= %lld and N <= %lld", (long long)kMaxG,
                (long long)kMaxN);
  if (!valid_k(K))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "K = %lld: need a multiple of 32 in [32, %lld]",
                (long long)K, (long long)kMaxK);
  ok();
  return G * matrix_bytes(N, K) + align256(4 * G);
}

int32_t nvfp4_pack(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t G,
                   int64_t N, int64_t K, void* packed, hipStream_t stream) {
  if (!codes || !scales || !g || !packed) return fail(NVFP4MOE_ERR_NULL_ARG, "nvfp4_pack: null");
  const int64_t bytes = nvfp4_packed_bytes(G, N, K);
  if (bytes < 0) return (int32_t)bytes;
  if (!aligned(packed, 16)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "packed must be 16-byte aligned");
  const int64_t chunks = G * tiles_per_matrix(N, K) * 512;
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(chunks, 256, 1 << 16)), dim3(256), 0, stream,
                     codes, scales, g, G, N, K, (uint8_t*)packed);
  return launched("nvfp4_pack");
}

int32_t nvfp4_dequant_f32(const void* packed, int64_t G, int64_t N, int64_t K, int32_t apply_g,
                          int32_t path, float* out, hipStream_t stream) {
  if (!packed || !out) return fail(NVFP4MOE_ERR_NULL_ARG, "nvfp4_dequant_f32: null");
  const int64_t bytes = nvfp4_packed_bytes(G, N, K);
  if (bytes < 0) return (int32_t)bytes;
  if (path != 0 && path != 1) return fail(NVFP4MOE_ERR_UNSUPPORTED, "path must be 0 or 1");
  if (!aligned(packed, 16)) return fail(NVFP4MOE_ERR_UNSUPPORTED, "packed must be 16-byte aligned");
  const int64_t chunks = G * tiles_per_matrix(N, K) * 512;
  hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(chunks, 256, 1 << 16)), dim3(256), 0, stream,
                     (const uint8_t*)packed, G, N, K, (int)apply_g, (int)path, out);
  return launched("nvfp4_dequant_f32");
}

int32_t nvfp4moe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words,
                             hipStream_t stream) {
  if (!src || !sink) return fail(NVFP4MOE_ERR_NULL_ARG, "nvfp4moe_stream_read: null");
  if (bytes < 16 || sink_words < 1) return fail(NVFP4MOE_ERR_BAD_SHAPE, "bytes >= 16, sink_words >= 1");
  if (bytes % 16 != 0 || !aligned(src, 16))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "bytes %% 16 == 0 and src 16-byte aligned");
  const int64_t n = bytes / 16;
  const int64_t blocks = nvfp4moe_stream_blocks(bytes);
  if (sink_words < blocks)
    return fail(NVFP4MOE_ERR_WORKSPACE, "sink needs %lld words", (long long)blocks);
  if (stream_unroll(bytes) == 1)
    hipLaunchKernelGGL(stream_read_kernel<1>, dim3((unsigned)blocks), dim3(kStreamThreads), 0,
                       stream, reinterpret_cast<const uint4*>(src), n, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)blocks), dim3(kStreamThreads), 0,
                       stream, reinterpret_cast<const uint4*>(src), n, sink);
  return launched("nvfp4moe_stream_read");
}

int64_t nvfp4moe_stream_blocks(int64_t bytes) {
  if (bytes < 16) return fail(NVFP4MOE_ERR_BAD_SHAPE, "bytes >= 16");
  ok();
  const int64_t per_block = (int64_t)kStreamThreads * stream_unroll(bytes);  // vectors per pass
  const int64_t want = (bytes / 16 + per_block - 1) / per_block;
  return want < kStreamMaxBlocks ? want : kStreamMaxBlocks;
}

int32_t nvfp4_quantize(const uint16_t* x, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                       uint8_t* scales, float* g, hipStream_t stream) {
  if (!x || !codes || !scales || !g) return fail(NVFP4MOE_ERR_NULL_ARG, "nvfp4_quantize: null");
  if (G < 1 || N < 1 || K < 16) return fail(NVFP4MOE_ERR_BAD_SHAPE, "G, N >= 1 and K >= 16");
  if (K % 16 != 0) return fail(NVFP4MOE_ERR_UNSUPPORTED, "K = %lld: need K %% 16 == 0", (long long)K);
  if (G > 65535) return fail(NVFP4MOE_ERR_UNSUPPORTED, "G = %lld > 65535", (long long)G);
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(g, 4))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "x 16-byte, codes 8-byte, g 4-byte aligned");
  const int64_t per = N * (K / 16);  // 16-element blocks per matrix
  const int64_t total = per * G;
  if ((total + kQuantThreads - 1) / kQuantThreads > ((int64_t)1 << 31) - 1)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "tensor too large");
  uint32_t* amax = reinterpret_cast<uint32_t*>(g);
  hipLaunchKernelGGL(quant_clear_kernel, dim3((unsigned)((G + kQuantThreads - 1) / kQuantThreads)),
                     dim3(kQuantThreads), 0, stream, amax, G);
  const int64_t bx = std::min<int64_t>((per + kQuantThreads - 1) / kQuantThreads,
                                       kQuantMaxBlocksPerMatrix);
  hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)bx, (unsigned)G), dim3(kQuantThreads), 0,
                     stream, x, per, amax);
  hipLaunchKernelGGL(quant_blocks_kernel,
                     dim3((unsigned)((per + kQuantThreads - 1) / kQuantThreads), (unsigned)G),
                     dim3(kQuantThreads), 0, stream, x, per, amax, codes, scales);
  hipLaunchKernelGGL(quant_finish_kernel, dim3((unsigned)((G + kQuantThreads - 1) / kQuantThreads)),
                     dim3(kQuantThreads), 0, stream, g, G);
  return launched("nvfp4_quantize");
}

int32_t nvfp4_skinny_gemm(const uint16_t* x, int64_t M, int64_t K, const void* w_packed,
                          int64_t N, uint16_t* y, hipStream_t stream) {
  if (!x || !w_packed || !y) return fail(NVFP4MOE_ERR_NULL_ARG, "nvfp4_skinny_gemm: null");
  if (M < 1 || N < 1) return fail(NVFP4MOE_ERR_BAD_SHAPE, "M and N must be >= 1");
  if (!valid_k(K))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "K = %lld: need a multiple of 32 in [32, %lld]",
                (long long)K, (long long)kMaxK);
  if (!aligned(x, 16) || !aligned(w_packed, 16))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "x and w_packed must be 16-byte aligned");
  if (K == 2048 && M >= kGemmDenseMinRows && M <= 16 &&
      (tiles_per_matrix(N, K) + 1) / 2 <= kGemmSplitKMaxBlocks) {
    const int64_t blocks16 = (tiles_per_matrix(N, K) + 1) / 2;
    hipLaunchKernelGGL(skinny_gemm_splitk_kernel, dim3((unsigned)blocks16),
                       dim3(64 * kGemmDenseWaves), 0, stream, x, M, (const uint8_t*)w_packed, N,
                       y);
    return launched("nvfp4_skinny_gemm");
  }
  if (K == 2048 && M >= kGemmDenseMinRows) {
    const int64_t blocks16 = (tiles_per_matrix(N, K) + 1) / 2;  // 16-row blocks of W
    const int64_t want = (blocks16 + kGemmDenseWaves - 1) / kGemmDenseWaves;
    const int64_t grid = want < kGemmDenseMaxBlocks ? want : kGemmDenseMaxBlocks;
    const size_t lds = (size_t)(M < 16 ? M : 16) * kGemmXStride;
    hipLaunchKernelGGL(skinny_gemm_dense_kernel, dim3((unsigned)grid),
                       dim3(64 * kGemmDenseWaves), lds, stream, x, M, (const uint8_t*)w_packed, N,
                       y);
    return launched("nvfp4_skinny_gemm");
  }
  if (row_blocks(N, K) > ((int64_t)1 << 32))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "N too large for the grid");
  return dispatch_l<GemmLaunch>(panel_k(K) / 32, x, M, K, (const uint8_t*)w_packed, N, y, stream);
}

int32_t fp8_skinny_gemm(const uint16_t* x, int64_t M, int64_t K, const uint8_t* w_fp8,
                        const float* scale, int64_t N, uint16_t* y, hipStream_t stream) {
  if (!x || !w_fp8 || !scale || !y) return fail(NVFP4MOE_ERR_NULL_ARG, "fp8_skinny_gemm: null");
  if (M < 1 || N < 1) return fail(NVFP4MOE_ERR_BAD_SHAPE, "M and N must be >= 1");
  if (K != 1024 && K != 2048 && K != 4096)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "K = %lld: need 1024, 2048 or 4096", (long long)K);
  if (!aligned(x, 16) || !aligned(w_fp8, 16))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "x and w_fp8 must be 16-byte aligned");
  const int64_t rpt = 8 / (K / 1024);
  const int64_t tiles = (N + rpt - 1) / rpt;
  if (tiles > ((int64_t)1 << 31) - 1) return fail(NVFP4MOE_ERR_UNSUPPORTED, "N too large");
  const dim3 grid((unsigned)tiles);
  switch (K) {
    case 1024:
      hipLaunchKernelGGL((fp8_skinny_gemm_kernel<1, 4>), grid, dim3(64), 0, stream, x, M, w_fp8,
                         scale, N, y);
      break;
    case 2048:
      hipLaunchKernelGGL((fp8_skinny_gemm_kernel<2, 4>), grid, dim3(64), 0, stream, x, M, w_fp8,
                         scale, N, y);
      break;
    default:
      hipLaunchKernelGGL((fp8_skinny_gemm_kernel<4, 4>), grid, dim3(64), 0, stream, x, M, w_fp8,
                         scale, N, y);
      break;
  }
  return launched("fp8_skinny_gemm");
}


int32_t moe_route_topk(const float* logits, const float* bias, int64_t M, int64_t E, int64_t k,
                       int32_t* ids, float* w, int32_t* counts, int32_t* offsets, int32_t* pairs,
                       int32_t* active, int32_t* active_offsets, int32_t* n_active,
                       hipStream_t stream) {
  const int32_t st = check_route(logits, M, E, k, ids, w, counts, offsets, pairs, active,
                                 active_offsets, n_active);
  if (st != NVFP4MOE_OK) return st;
  return launch_route(logits, bias, M, E, k, ids, w, counts, offsets, pairs, active,
                      active_offsets, n_active, stream);
}

int32_t moe_route_project_topk(const uint16_t* x, const uint16_t* w_router, const float* bias,
                               int64_t M, int64_t E, int64_t k, int64_t H, float* logits,
                               int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                               int32_t* pairs, int32_t* active, int32_t* active_offsets,
                               int32_t* n_active, hipStream_t stream) {
  if (!x || !w_router) return fail(NVFP4MOE_ERR_NULL_ARG, "moe_route_project_topk: null");
  int32_t st = check_route(logits, M, E, k, ids, w, counts, offsets, pairs, active,
                           active_offsets, n_active);
  if (st != NVFP4MOE_OK) return st;
  if (H != 512 && H != 1024 && H != 2048 && H != 4096)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "H = %lld: need 512, 1024, 2048 or 4096",
                (long long)H);
  if (!aligned(x, 16) || !aligned(w_router, 16))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "x and w_router must be 16-byte aligned");
  const dim3 grid((unsigned)E), block(256);
  switch (H) {
    case 512:
      hipLaunchKernelGGL(router_logits_kernel<2>, grid, block, 0, stream, x, M, w_router, (int)E,
                         logits);
      break;
    case 1024:
      hipLaunchKernelGGL(router_logits_kernel<4>, grid, block, 0, stream, x, M, w_router, (int)E,
                         logits);
      break;
    case 2048:
      hipLaunchKernelGGL(router_logits_kernel<8>, grid, block, 0, stream, x, M, w_router, (int)E,
                         logits);
      break;
    default:
      hipLaunchKernelGGL(router_logits_kernel<16>, grid, block, 0, stream, x, M, w_router, (int)E,
                         logits);
      break;
  }
  st = launched("moe_route_project_topk logits");
  if (st != NVFP4MOE_OK) return st;
  return launch_route(logits, bias, M, E, k, ids, w, counts, offsets, pairs, active,
                      active_offsets, n_active, stream);
}

int64_t moe_nvfp4_workspace_bytes(int64_t M, int64_t E, int64_t k, int64_t H, int64_t I,
                                  int32_t has_shared) {
  if (M < 1 || E < 1 || k < 1 || H < 1 || I < 1)
    return fail(NVFP4MOE_ERR_BAD_SHAPE, "sizes must be >= 1");
  if (!valid_k(H) || !valid_k(I))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "H and I must be multiples of 32 in [32, %lld]",
                (long long)kMaxK);
  ok();
  return ws_layout(M, k, H, I, has_shared != 0).total;
}

int32_t moe_nvfp4_decode(const moe_nvfp4_args* a, hipStream_t stream) {
  MoeParams p;
  const int32_t st = prepare_decode(a, true, p);
  if (st != NVFP4MOE_OK) return st;
  if (a->proj_w)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "the projection rides on moe_nvfp4_route_decode only");
  const int64_t M = a->M, H = a->H, I = a->I;
  const bool specialised = H == 2048 && I == 512;
  // the specialised kernels take 64 gate and 64 down row blocks as constants
  if (specialised && (p.PG != 64 || p.PD != 64))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "internal: row blocks %d / %d", p.PG, p.PD);
  // per-row down + combine needs FP32 h for every pair: no slot (the shared
  // one has M rows) may take the MFMA gate_up path
  const bool valu_h = M < p.dense_min_rows || !specialised;
  if (a->schedule == 3 && !valu_h)
    return fail(NVFP4MOE_ERR_UNSUPPORTED,
                "schedule 3 needs M < dense_min_rows (FP32 h for every pair)");
  const bool token_major =
      a->schedule == 3 || (a->schedule == 0 && valu_h && M <= kTokenMajorMaxRows);
  // one row per batch keeps these kernels at three waves per SIMD; slots
  // with many rows go to MFMA (specialised shapes) or take more batches
  const int rmax_s = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  return launch_staged_rows(p, specialised, rmax_s, token_major, stream);
}

}  // extern "C"

namespace {

// moe_nvfp4_route_decode with its h rows in `scratch` (scratch_bytes) when
// not null, else in the caller's workspace.
int32_t route_decode(const moe_nvfp4_args* a, const float* logits, const float* bias,
                     hipStream_t stream, void* scratch, int64_t scratch_bytes) {
  if (!logits) return fail(NVFP4MOE_ERR_NULL_ARG, "moe_nvfp4_route_decode: logits is null");
  MoeParams p;
  const int32_t st = prepare_decode(a, false, p, scratch, scratch_bytes);
  if (st != NVFP4MOE_OK) return st;
  const int64_t M = a->M, H = a->H, I = a->I;
  const bool specialised = H == 2048 && I == 512;
  // the specialised kernels take 64 gate and 64 down row blocks as constants
  if (specialised && (p.PG != 64 || p.PD != 64))
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "internal: row blocks %d / %d", p.PG, p.PD);
  if (specialised && M >= p.dense_min_rows)
    return fail(NVFP4MOE_ERR_UNSUPPORTED,
                "moe_nvfp4_route_decode needs M < dense_min_rows (FP32 h for every pair)");
  if (a->proj_w) {
    if (!a->proj_out) return fail(NVFP4MOE_ERR_NULL_ARG, "proj_out is null");
    if (a->proj_n < 1) return fail(NVFP4MOE_ERR_BAD_SHAPE, "proj_n must be >= 1");
    if (H != 2048 || M > 16 || a->proj_n > 4096 || a->k + p.has_shared < 4)
      return fail(NVFP4MOE_ERR_UNSUPPORTED,
                  "projection: needs H = 2048, M <= 16, proj_n <= 4096, k (+ shared) >= 4");
    if (!aligned(a->proj_w, 16) || !aligned(a->proj_out, 16))
      return fail(NVFP4MOE_ERR_UNSUPPORTED, "proj_w and proj_out must be 16-byte aligned");
    // the projection's blocks read x while the other blocks of the same launch
    // write out (and the projection blocks write proj_out)
    const int64_t xb = M * H * 2;
    if (overlaps(a->x, xb, a->out, xb) || overlaps(a->x, xb, a->proj_out, M * a->proj_n * 2))
      return fail(NVFP4MOE_ERR_BAD_SHAPE,
                  "with a projection, out and proj_out must not overlap x (residual == out is "
                  "fine)");
    p.pw = static_cast<const uint8_t*>(a->proj_w);
    p.py = a->proj_out;
    p.pn = a->proj_n;
    const int64_t blocks16 = (tiles_per_matrix(a->proj_n, 2048) + 1) / 2;
    p.proj_blocks = (int)((blocks16 + 7) / 8 * 8);  // keeps the down blocks' XCD order
  }
  const int grid = (int)((M * a->k + (p.has_shared ? M : 0)) * p.PG);
  int32_t* ids = const_cast<int32_t*>(a->ids);
  float* w = const_cast<float*>(a->w);
  if (specialised && p.has_shared)
    hipLaunchKernelGGL((fused_route_gate_kernel<64, true>), dim3(grid), dim3(128), 0, stream, p,
                       logits, bias, ids, w);
  else if (specialised)
    hipLaunchKernelGGL((fused_route_gate_kernel<64, false>), dim3(grid), dim3(128), 0, stream, p,
                       logits, bias, ids, w);
  else if (p.has_shared)
    hipLaunchKernelGGL((fused_route_gate_kernel<0, true>), dim3(grid), dim3(128), 0, stream, p,
                       logits, bias, ids, w);
  else
    hipLaunchKernelGGL((fused_route_gate_kernel<0, false>), dim3(grid), dim3(128), 0, stream, p,
                       logits, bias, ids, w);
  const int32_t st2 = launched("moe_nvfp4_route_decode gate_up");
  if (st2 != NVFP4MOE_OK) return st2;
  if (specialised)
    launch_token_down<16>(p, stream);
  else
    launch_token_down<0>(p, stream);
  return launched("moe_nvfp4_route_decode");
}

// ---- scratch for the call that allocates nothing --------------------------------------

std::mutex g_scratch_mu;
void* g_scratch[kScratchMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device (each GPU holds its own copy at its own address).
int32_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NVFP4MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchMaxDevices)
    return fail(NVFP4MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
                kScratchMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(NVFP4MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return ok();
}

}  // namespace

extern "C" {

int32_t moe_nvfp4_route_decode(const moe_nvfp4_args* a, const float* logits, const float* bias,
                               hipStream_t stream) {
  return route_decode(a, logits, bias, stream, nullptr, 0);
}

int32_t moe_nvfp4_route_decode_static(const moe_nvfp4_args* a, const float* logits,
                                      const float* bias, hipStream_t stream) {
  if (!a) return fail(NVFP4MOE_ERR_NULL_ARG, "moe_nvfp4_route_decode_static: args is null");
  if (a->M >= 1 && a->k >= 1 && a->H >= 1 && a->I >= 1) {
    const int64_t need = ws_layout(a->M, a->k, a->H, a->I, a->shared_gate_up != nullptr).yp_off;
    if (need > kScratchBytes)
      return fail(NVFP4MOE_ERR_UNSUPPORTED,
                  "h rows need %lld bytes of scratch; the static scratch holds %lld",
                  (long long)need, (long long)kScratchBytes);
  }
  void* ptr = nullptr;
  const int32_t st = scratch_address(&ptr);
  if (st != NVFP4MOE_OK) return st;
  return route_decode(a, logits, bias, stream, ptr, kScratchBytes);
}

}  // extern "C"
