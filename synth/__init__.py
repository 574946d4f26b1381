"""Seeded synthetic inputs for the NVFP4 MoE decode path.

Thin numpy wrapper over libsynth.so (synth.c). The generator holds none of
the method's arithmetic: it emits canonical input bytes that both the
float64 oracle and the GPU library consume unchanged.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

_u64 = ctypes.c_uint64
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_mix.restype = _u64
        L.synth_mix.argtypes = [_u64]
        L.synth_key.restype = _u64
        L.synth_key.argtypes = [_u64] * 5
        L.synth_u64.restype = _u64
        L.synth_u64.argtypes = [_u64, _u64]
        L.synth_fill_bytes.restype = None
        L.synth_fill_bytes.argtypes = [_u64, _vp, _i64, ctypes.c_int]
        L.synth_fill_scales.restype = ctypes.c_int
        L.synth_fill_scales.argtypes = [_u64, _vp, _i64, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_int]
        L.synth_fill_normal_f32.restype = None
        L.synth_fill_normal_f32.argtypes = [_u64, _vp, _i64, ctypes.c_double, ctypes.c_double]
        L.synth_fill_normal_bf16.restype = None
        L.synth_fill_normal_bf16.argtypes = [_u64, _vp, _i64, ctypes.c_double, ctypes.c_double]
        L.synth_fill_zipf_gumbel.restype = None
        L.synth_fill_zipf_gumbel.argtypes = [_u64, _u64, _vp, _i64, _i64, ctypes.c_double]
        L.synth_fill_bytes_keys.restype = None
        L.synth_fill_bytes_keys.argtypes = [_vp, _i64, _vp, _i64, ctypes.c_int]
        L.synth_fill_scales_keys.restype = ctypes.c_int
        L.synth_fill_scales_keys.argtypes = [_vp, _i64, _vp, _i64, ctypes.c_double,
                                             ctypes.c_double, ctypes.c_int]
        _lib = L
    return _lib


def key(seed, a=0, b=0, c=0, d=0) -> int:
    return int(lib().synth_key(seed, a, b, c, d))


def u64(k, i) -> int:
    return int(lib().synth_u64(k, i))


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(_vp)


def uniform_bytes(k, shape, nthreads=0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint8)
    lib().synth_fill_bytes(k, _ptr(out), out.size, nthreads)
    return out


def scale_codes(k, shape, lo_log2=-4.0, hi_log2=4.0, nthreads=0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint8)
    rc = lib().synth_fill_scales(k, _ptr(out), out.size, lo_log2, hi_log2, nthreads)
    if rc != 0:
        raise ValueError("scale range must satisfy -6 <= lo < hi <= 8")
    return out


def normal_f32(k, shape, mean=0.0, std=1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    lib().synth_fill_normal_f32(k, _ptr(out), out.size, mean, std)
    return out


def normal_bf16(k, shape, mean=0.0, std=1.0) -> np.ndarray:
    """BF16 bit patterns (uint16) of N(mean, std^2) samples."""
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_fill_normal_bf16(k, _ptr(out), out.size, mean, std)
    return out


def zipf_gumbel_logits(k, perm_k, M, E, s) -> np.ndarray:
    out = np.empty((M, E), dtype=np.float32)
    lib().synth_fill_zipf_gumbel(k, perm_k, _ptr(out), M, E, s)
    return out


def uniform_bytes_keys(keys, per, nthreads=0) -> np.ndarray:
    """[len(keys)][per] bytes, row g drawn from stream keys[g]."""
    ks = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
    out = np.empty((len(ks), per), dtype=np.uint8)
    lib().synth_fill_bytes_keys(_ptr(ks), len(ks), _ptr(out), per, nthreads)
    return out


def scale_codes_keys(keys, per, lo_log2=-4.0, hi_log2=4.0, nthreads=0) -> np.ndarray:
    ks = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
    out = np.empty((len(ks), per), dtype=np.uint8)
    rc = lib().synth_fill_scales_keys(_ptr(ks), len(ks), _ptr(out), per, lo_log2, hi_log2,
                                      nthreads)
    if rc != 0:
        raise ValueError("scale range must satisfy -6 <= lo < hi <= 8")
    return out
