"""float64 CPU oracle for the NVFP4 MoE decode path (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg. The GPU library and its Python binding never
import it. Functions take and return numpy arrays in the canonical layouts
documented in oracle.h.

The products and the MoE block split their outputs over threads (results are
bit-identical for every thread count): by default the CPUs this process may
run on, at most 16, or NVFP4MOE_ORACLE_THREADS if set; set_threads() changes
it.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_vp, _i64 = ctypes.c_void_p, ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e2m1.restype = ctypes.c_double
        L.oracle_e2m1.argtypes = [ctypes.c_uint32]
        L.oracle_e4m3.restype = ctypes.c_double
        L.oracle_e4m3.argtypes = [ctypes.c_uint32]
        L.oracle_bf16.restype = ctypes.c_double
        L.oracle_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp]
        L.oracle_dequant_f32.restype = None
        L.oracle_dequant_f32.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp]
        L.oracle_gemm.restype = None
        L.oracle_gemm.argtypes = [_vp, _i64, _i64, _vp, _vp, ctypes.c_float, _i64, _vp]
        L.oracle_gemm_fp8.restype = None
        L.oracle_gemm_fp8.argtypes = [_vp, _i64, _i64, _vp, ctypes.c_double, _i64, _vp]
        L.oracle_quantize_nvfp4.restype = None
        L.oracle_quantize_nvfp4.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp]
        L.oracle_e4m3_rne.restype = ctypes.c_uint32
        L.oracle_e4m3_rne.argtypes = [ctypes.c_float]
        L.oracle_e2m1_rne.restype = ctypes.c_uint32
        L.oracle_e2m1_rne.argtypes = [ctypes.c_float]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp]
        L.oracle_route_topk.restype = ctypes.c_int
        L.oracle_route_topk.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp]
        L.oracle_group_by_expert.restype = None
        L.oracle_group_by_expert.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [_vp, _i64, _i64, _vp, _vp, ctypes.c_float, _vp, _vp,
                                        ctypes.c_float, _vp]
        L.oracle_moe_block.restype = None
        L.oracle_moe_block.argtypes = [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp] + [_vp] * 13
        L.oracle_moe_block_f64.restype = None
        L.oracle_moe_block_f64.argtypes = [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp] + \
            [_vp] * 13
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_threads.argtypes = []
        L.oracle_set_threads(default_threads())
        L.oracle_moe_decode.restype = ctypes.c_int
        L.oracle_moe_decode.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64] + \
            [_vp] * 16
        _lib = L
    return _lib


def default_threads() -> int:
    env = os.environ.get("NVFP4MOE_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def threads() -> int:
    return int(lib().oracle_threads())


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous, "need a C-contiguous ndarray"
    return a.ctypes.data_as(_vp)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e4m3(byte: int) -> float:
    return lib().oracle_e4m3(byte)


def bf16(bits: int) -> float:
    return lib().oracle_bf16(bits)


def dequant(codes, scales, g) -> np.ndarray:
    codes, scales, g = _c(codes, np.uint8), _c(scales, np.uint8), _c(g, np.float32)
    G, N, kh = codes.shape
    out = np.empty((G, N, kh * 2), dtype=np.float64)
    lib().oracle_dequant(_p(codes), _p(scales), _p(g), G, N, kh * 2, _p(out))
    return out


def dequant_f32(codes, scales, g) -> np.ndarray:
    codes, scales, g = _c(codes, np.uint8), _c(scales, np.uint8), _c(g, np.float32)
    G, N, kh = codes.shape
    out = np.empty((G, N, kh * 2), dtype=np.float32)
    lib().oracle_dequant_f32(_p(codes), _p(scales), _p(g), G, N, kh * 2, _p(out))
    return out


def gemm(x_bf16, codes, scales, g) -> np.ndarray:
    """x: uint16 [M][K]; codes [N][K/2] (or [1][N][K/2]); returns float64 [M][N]."""
    x = _c(x_bf16, np.uint16)
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    M, K = x.shape
    N = codes.shape[-2]
    assert codes.shape[-1] * 2 == K
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm(_p(x), M, K, _p(codes), _p(scales), float(np.float32(g)), N, _p(y))
    return y


def gemm_fp8(x_bf16, w_fp8, s) -> np.ndarray:
    """x: uint16 [M][K]; w_fp8: uint8 E4M3 codes [N][K]; s: tensor scale.
    Returns float64 [M][N]."""
    x, w = _c(x_bf16, np.uint16), _c(w_fp8, np.uint8)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm_fp8(_p(x), M, K, _p(w), float(s), N, _p(y))
    return y


def quantize_nvfp4(x_bf16):
    """x: uint16 BF16 bits [G][N][K] (or [N][K]) -> (codes uint8 [G][N][K/2],
    scales uint8 [G][N][K/16], g float32 [G]) by the amax recipe of oracle.cpp."""
    x = _c(x_bf16, np.uint16)
    if x.ndim == 2:
        x = x[None]
    G, N, K = x.shape
    assert K % 16 == 0
    codes = np.empty((G, N, K // 2), np.uint8)
    scales = np.empty((G, N, K // 16), np.uint8)
    g = np.empty(G, np.float32)
    lib().oracle_quantize_nvfp4(_p(x), G, N, K, _p(codes), _p(scales), _p(g))
    return codes, scales, g


def e4m3_rne(t: float) -> int:
    return int(lib().oracle_e4m3_rne(t))


def e2m1_rne(v: float) -> int:
    return int(lib().oracle_e2m1_rne(v))


def router_logits(x_bf16, w_router_bf16) -> np.ndarray:
    """x: uint16 [M][H]; w_router: uint16 [E][H] (BF16 bits). Returns float64
    [M][E] = x W_r^T."""
    x, wr = _c(x_bf16, np.uint16), _c(w_router_bf16, np.uint16)
    M, H = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == H
    out = np.empty((M, E), dtype=np.float64)
    lib().oracle_router_logits(_p(x), M, H, _p(wr), E, _p(out))
    return out


def route_topk(logits, k, bias=None):
    lg = _c(logits, np.float32)
    M, E = lg.shape
    b = _c(bias, np.float32)
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float64)
    rc = lib().oracle_route_topk(_p(lg), _p(b), M, E, k, _p(ids), _p(w))
    if rc != 0:
        raise ValueError("k must satisfy 1 <= k <= E")
    return ids, w


def group_by_expert(ids, E):
    ids = _c(ids, np.int32)
    M, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    pairs = np.empty(M * k, np.int32)
    active = np.empty(E, np.int32)
    active_offsets = np.empty(E + 1, np.int32)
    na = np.zeros(1, np.int32)
    lib().oracle_group_by_expert(_p(ids), M, E, k, _p(counts), _p(offsets), _p(pairs),
                                 _p(active), _p(active_offsets), _p(na))
    return counts, offsets, pairs, active, active_offsets, int(na[0])


def expert_ffn(x_row, gate_up, down):
    """gate_up / down: NVFP4 with G == 1."""
    x = _c(x_row, np.uint16)
    H = x.shape[-1]
    I = down.codes.shape[-1] * 2
    y = np.empty(H, dtype=np.float64)
    lib().oracle_expert_ffn(_p(x), H, I, _p(_c(gate_up.codes, np.uint8)),
                            _p(_c(gate_up.scales, np.uint8)), float(gate_up.g[0]),
                            _p(_c(down.codes, np.uint8)), _p(_c(down.scales, np.uint8)),
                            float(down.g[0]), _p(y))
    return y


def _shared_ptrs(sgu, sdn):
    if sgu is None:
        return [None] * 6, []
    keep = [_c(sgu.codes, np.uint8), _c(sgu.scales, np.uint8), _c(sgu.g, np.float32),
            _c(sdn.codes, np.uint8), _c(sdn.scales, np.uint8), _c(sdn.g, np.float32)]
    return [_p(a) for a in keep], keep


def moe_block(x, ids, w, gate_up, down, shared_gate_up=None, shared_down=None, residual=None):
    """out float64 [M][H] = sum_j w * ffn(x) (+ shared) (+ residual).
    ids index into gate_up/down's leading (expert) axis."""
    x = _c(x, np.uint16)
    ids, w = _c(ids, np.int32), _c(w, np.float64)
    M, H = x.shape
    k = ids.shape[1]
    E = gate_up.codes.shape[0]
    I = down.codes.shape[-1] * 2
    gu = [_c(gate_up.codes, np.uint8), _c(gate_up.scales, np.uint8), _c(gate_up.g, np.float32)]
    dn = [_c(down.codes, np.uint8), _c(down.scales, np.uint8), _c(down.g, np.float32)]
    sh, keep = _shared_ptrs(shared_gate_up, shared_down)
    res = _c(residual, np.uint16)
    out = np.empty((M, H), dtype=np.float64)
    lib().oracle_moe_block(_p(x), M, H, I, E, k, _p(ids), _p(w), *[_p(a) for a in gu],
                           *[_p(a) for a in dn], *sh, _p(res), _p(out))
    del keep
    return out


def moe_block_f64(x, ids, w, gate_up, down, shared_gate_up=None, shared_down=None,
                  residual=None):
    """moe_block with x [M][H] and residual given as float64 values (the
    float64 chain of a layer stack)."""
    x = _c(x, np.float64)
    ids, w = _c(ids, np.int32), _c(w, np.float64)
    M, H = x.shape
    k = ids.shape[1]
    E = gate_up.codes.shape[0]
    I = down.codes.shape[-1] * 2
    gu = [_c(gate_up.codes, np.uint8), _c(gate_up.scales, np.uint8), _c(gate_up.g, np.float32)]
    dn = [_c(down.codes, np.uint8), _c(down.scales, np.uint8), _c(down.g, np.float32)]
    sh, keep = _shared_ptrs(shared_gate_up, shared_down)
    res = _c(residual, np.float64)
    out = np.empty((M, H), dtype=np.float64)
    lib().oracle_moe_block_f64(_p(x), M, H, I, E, k, _p(ids), _p(w), *[_p(a) for a in gu],
                               *[_p(a) for a in dn], *sh, _p(res), _p(out))
    del keep
    return out


def moe_block_touched(layer, ids, w, rows=None, residual=None):
    """moe_block over only the experts that ids touches (for large expert
    sets): selects those experts and remaps ids. rows: optional subset."""
    ids = np.asarray(ids, dtype=np.int32)
    x = layer.x
    if rows is not None:
        rows = np.asarray(rows)
        ids, w, x = ids[rows], np.asarray(w)[rows], x[rows]
        residual = None if residual is None else np.asarray(residual)[rows]
    used = np.unique(ids)
    remap = np.full(layer.E, -1, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    return moe_block(x, remap[ids], w, layer.gate_up.select(used), layer.down.select(used),
                     layer.shared_gate_up, layer.shared_down, residual)


def moe_decode(x, logits, k, gate_up, down, bias=None, shared_gate_up=None, shared_down=None,
               residual=None):
    """The whole step from logits: returns (ids, w, out)."""
    x = _c(x, np.uint16)
    lg = _c(logits, np.float32)
    M, H = x.shape
    E = lg.shape[1]
    I = down.codes.shape[-1] * 2
    gu = [_c(gate_up.codes, np.uint8), _c(gate_up.scales, np.uint8), _c(gate_up.g, np.float32)]
    dn = [_c(down.codes, np.uint8), _c(down.scales, np.uint8), _c(down.g, np.float32)]
    sh, keep = _shared_ptrs(shared_gate_up, shared_down)
    res = _c(residual, np.uint16)
    b = _c(bias, np.float32)
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float64)
    out = np.empty((M, H), np.float64)
    rc = lib().oracle_moe_decode(_p(x), _p(lg), _p(b), M, H, I, E, k, *[_p(a) for a in gu],
                                 *[_p(a) for a in dn], *sh, _p(res), _p(ids), _p(w), _p(out))
    del keep
    if rc != 0:
        raise ValueError("bad routing arguments")
    return ids, w, out
