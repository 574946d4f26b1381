"""Seeded synthetic workloads for the NVFP4 MoE decode path.

Every tensor is in the canonical NVFP4 layout that both the oracle and the
GPU library accept:
  codes  uint8 [G][N][K/2]   E2M1 codes, element 2b in the low nibble of byte b
  scales uint8 [G][N][K/16]  E4M3 code per 16 consecutive elements along K
  g      float32 [G]         per-matrix FP32 tensor scale
A weight matrix is stored [N][K] (out x in) and applied as y = x W^T.

Recipe (per tensor a SplitMix64 stream keyed by seed, workload, layer, tensor
and expert): activations BF16(N(0,1)); router logits FP32 N(0,1); codes
uniform over all 16 E2M1 codes; scales E4M3(2^U[-4,4)); tensor scale 1.0 for
the single dense matrix and 2^-9 (K = 2048) / 2^-8 (K = 512) elsewhere, which
keeps every activation O(1) through a residual chain.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import key, normal_bf16, normal_f32, scale_codes_keys, uniform_bytes, uniform_bytes_keys, \
    zipf_gumbel_logits

# tensor identifiers inside a stream key
T_X, T_LOGITS, T_BIAS = 1, 2, 3
T_GU_CODES, T_GU_SCALES, T_DN_CODES, T_DN_SCALES = 4, 5, 6, 7
T_SH_GU_CODES, T_SH_GU_SCALES, T_SH_DN_CODES, T_SH_DN_SCALES = 8, 9, 10, 11
T_P_CODES, T_P_SCALES, T_PERM, T_W_CODES, T_W_SCALES = 12, 13, 14, 15, 16
T_ROUTER = 17

H, I, E, TOPK = 2048, 512, 256, 8
G_K2048 = 2.0 ** -9
G_K512 = 2.0 ** -8


def tensor_scale_for_k(K: int) -> float:
    """2^round(log2(1/sqrt(K * E[v^2 s^2]))) with E[v^2 s^2] ~ 198: 2^-9 at K=2048,
    2^-8 at K=512. Keeps x W^T at unit scale for unit-variance x."""
    import math
    return 2.0 ** round(math.log2(1.0 / math.sqrt(K * 198.0)))


@dataclass
class NVFP4:
    codes: np.ndarray   # uint8 [G][N][K/2]
    scales: np.ndarray  # uint8 [G][N][K/16]
    g: np.ndarray       # float32 [G]

    @property
    def shape(self):
        G, N, kh = self.codes.shape
        return G, N, kh * 2

    def select(self, idx) -> "NVFP4":
        idx = np.asarray(idx)
        return NVFP4(np.ascontiguousarray(self.codes[idx]), np.ascontiguousarray(self.scales[idx]),
                     np.ascontiguousarray(self.g[idx]))


def nvfp4_random(seed, wl, layer, t_codes, t_scales, G, N, K, g, experts=None) -> NVFP4:
    """G matrices [N][K]; matrix e uses its own streams, so a subset of experts
    regenerates bit-identically on its own."""
    ids = range(G) if experts is None else experts
    kc = [key(seed, wl, layer, t_codes, e) for e in ids]
    ks = [key(seed, wl, layer, t_scales, e) for e in ids]
    codes = uniform_bytes_keys(kc, N * K // 2).reshape(len(kc), N, K // 2)
    scales = scale_codes_keys(ks, N * K // 16).reshape(len(ks), N, K // 16)
    return NVFP4(codes, scales, np.full(len(kc), g, dtype=np.float32))


@dataclass
class MoELayer:
    M: int
    H: int
    I: int
    E: int
    k: int
    x: np.ndarray                 # uint16 (bf16 bits) [M][H]
    logits: np.ndarray            # float32 [M][E]
    bias: Optional[np.ndarray]    # float32 [E] or None
    gate_up: NVFP4                # [E][2I][H]  rows 0..I-1 gate, I..2I-1 up
    down: NVFP4                   # [E][H][I]
    shared_gate_up: Optional[NVFP4] = None  # [1][2I][H]
    shared_down: Optional[NVFP4] = None     # [1][H][I]
    extra: dict = field(default_factory=dict)


def moe_layer(seed=0, wl=2, layer=0, M=4, E_=E, H_=H, I_=I, k=TOPK, bias=False,
              shared=False, zipf_s=None, x=None, g_gu=None, g_dn=None,
              bias_std=0.5) -> MoELayer:
    if x is None:
        x = normal_bf16(key(seed, wl, layer, T_X, 0), (M, H_))
    if zipf_s is None:
        logits = normal_f32(key(seed, wl, layer, T_LOGITS, 0), (M, E_))
    else:
        logits = zipf_gumbel_logits(key(seed, wl, layer, T_LOGITS, 0),
                                    key(seed, wl, layer, T_PERM, 0), M, E_, zipf_s)
    b = normal_f32(key(seed, wl, layer, T_BIAS, 0), (E_,), 0.0, bias_std) if bias else None
    g_gu = tensor_scale_for_k(H_) if g_gu is None else g_gu
    g_dn = tensor_scale_for_k(I_) if g_dn is None else g_dn
    gu = nvfp4_random(seed, wl, layer, T_GU_CODES, T_GU_SCALES, E_, 2 * I_, H_, g_gu)
    dn = nvfp4_random(seed, wl, layer, T_DN_CODES, T_DN_SCALES, E_, H_, I_, g_dn)
    sgu = sdn = None
    if shared:
        sgu = nvfp4_random(seed, wl, layer, T_SH_GU_CODES, T_SH_GU_SCALES, 1, 2 * I_, H_, g_gu)
        sdn = nvfp4_random(seed, wl, layer, T_SH_DN_CODES, T_SH_DN_SCALES, 1, H_, I_, g_dn)
    return MoELayer(M, H_, I_, E_, k, x, logits, b, gu, dn, sgu, sdn)


# ---- the five workloads -------------------------------------------------------

def dense_skinny(seed=0, M=1, K=2048, N=512, g=1.0, wl=1, layer=0, t_codes=T_W_CODES,
                 t_scales=T_W_SCALES, x=None):
    """One dense NVFP4 matrix [N][K] and M BF16 rows: the skinny projection."""
    if x is None:
        x = normal_bf16(key(seed, wl, layer, T_X, 0), (M, K))
    w = nvfp4_random(seed, wl, layer, t_codes, t_scales, 1, N, K, g)
    return x, w


def draft_head(seed=0, M=6, N=32768, layer=0):
    """A large-N skinny projection: M BF16 rows (a token and its draft tokens)
    times a [N][2048] NVFP4 head, tensor scale 2^-9 (unit-scale outputs)."""
    return dense_skinny(seed, M=M, K=H, N=N, g=tensor_scale_for_k(H), wl=6, layer=layer)


def fp8_projection(seed=0, M=4, K=2048, N=5120, layer=0):
    """M BF16 rows and an FP8 E4M3 matrix [N][K] with one tensor scale: the
    attention-projection product. Codes: random sign, exponent field 4..11,
    random mantissa (values 2^-3 .. 30, never NaN); scale 2^round(-log2(
    sqrt(K E[v^2]))) with E[v^2] = 2.1484 * 42.66 for this code distribution,
    so that outputs are of unit scale."""
    x = normal_bf16(key(seed, 7, layer, T_X, 0), (M, K))
    b = uniform_bytes(key(seed, 7, layer, T_W_CODES, 0), (N, K))
    sign = uniform_bytes(key(seed, 7, layer, T_W_SCALES, 0), (N, K)) & 0x80
    codes = (sign | ((4 + ((b >> 3) & 7)) << 3) | (b & 7)).astype(np.uint8)
    s = 2.0 ** round(-np.log2(np.sqrt(K * 2.1484375 * 42.666)))
    return x, codes, float(s)


def router_weights(seed=0, wl=2, layer=0, E_=E, H_=H):
    """BF16 router matrix [E][H], entries N(0, 1/H): for rows of unit RMS the
    logits x W_r^T are about N(0, 1), the logit scale of the other workloads."""
    return normal_bf16(key(seed, wl, layer, T_ROUTER, 0), (E_, H_), 0.0, 1.0 / np.sqrt(H_))


def decode_m4(seed=0):
    """One MoE block, 4 rows (one token plus three draft tokens verified together)."""
    return moe_layer(seed, wl=2, M=4)


def decode_m16_shared(seed=0):
    """One MoE block, 16 rows, per-expert logit bias N(0, 0.5^2), plus one
    always-on shared expert."""
    return moe_layer(seed, wl=3, M=16, bias=True, shared=True)


STACK_LAYERS = 40
STACK_M = 8
STACK_PROJ_N = 64
# The block's output is quadratic in its input (silu(u) * u), so a residual
# chain x + moe(x) with unit-gain blocks diverges within a few layers. The
# stack's down projections (routed and shared) use a 16x smaller tensor scale,
# which keeps the 40-layer chain at O(1) (rms 1.0 -> ~1.2).
STACK_G_DOWN = 2.0 ** -12


def stack_layer(l, seed=0, x=None):
    """Layer l of the 40-block stack at 8 rows: routed experts + shared expert,
    logits N(0,1) per layer, plus a dense NVFP4 2048->64 projection."""
    lay = moe_layer(seed, wl=4, layer=l, M=STACK_M, shared=True, x=x, g_dn=STACK_G_DOWN)
    _, proj = dense_skinny(seed, M=STACK_M, K=H, N=STACK_PROJ_N, g=G_K2048, wl=4, layer=l,
                           t_codes=T_P_CODES, t_scales=T_P_SCALES, x=lay.x)
    lay.extra["proj"] = proj
    return lay


def stack_x0(seed=0):
    return normal_bf16(key(seed, 4, 0, T_X, 0), (STACK_M, H))


def prefill_m256(seed=0):
    """A 256-row chunk through one MoE block with Zipf(1.1) expert popularity."""
    return moe_layer(seed, wl=5, M=256, zipf_s=1.1)
