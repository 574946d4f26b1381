"""nvfp4_moe_skinny_amd: Python binding of libnvfp4moe.so.

Argument marshalling only. Every computation runs in the library's HIP
kernels on the GPU; PyTorch supplies device memory and the current stream.
There is no CPU fallback: if the library is missing, importing the binding
raises.

The functions carry the C names (see include/nvfp4moe.h for the contract)
and take torch tensors on the GPU in the documented dtypes and layouts.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4moe.so")

NVFP4MOE_OK = 0
NVFP4MOE_ERR_NULL_ARG = -1
NVFP4MOE_ERR_BAD_SHAPE = -2
NVFP4MOE_ERR_UNSUPPORTED = -3
NVFP4MOE_ERR_WORKSPACE = -4
NVFP4MOE_ERR_HIP = -5

_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32


class NVFP4MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {strerror(status)} ({detail})")
        self.status = status


class MoeArgs(ctypes.Structure):
    """Mirror of struct moe_nvfp4_args."""
    _fields_ = [
        ("x", _vp), ("ids", _vp), ("w", _vp), ("offsets", _vp), ("pairs", _vp),
        ("active", _vp), ("active_offsets", _vp), ("n_active", _vp), ("w_gate_up", _vp),
        ("w_down", _vp),
        ("shared_gate_up", _vp), ("shared_down", _vp), ("residual", _vp), ("out", _vp),
        ("workspace", _vp), ("workspace_bytes", _i64),
        ("M", _i64), ("E", _i64), ("k", _i64), ("H", _i64), ("I", _i64),
        ("dense_min_rows", _i64), ("schedule", _i32),
        ("proj_w", _vp), ("proj_n", _i64), ("proj_out", _vp),
    ]

# moe_nvfp4_args.schedule
SCHEDULE_AUTO, SCHEDULE_THREE_LAUNCHES, SCHEDULE_TWO_LAUNCHES = 0, 2, 3


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python nvfp4_moe_skinny_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    L.nvfp4moe_strerror.restype = ctypes.c_char_p
    L.nvfp4moe_strerror.argtypes = [_i32]
    L.nvfp4moe_last_error_detail.restype = ctypes.c_char_p
    L.nvfp4moe_last_error_detail.argtypes = []
    L.nvfp4moe_version.restype = ctypes.c_char_p
    L.nvfp4moe_version.argtypes = []
    L.nvfp4_packed_bytes.restype = _i64
    L.nvfp4_packed_bytes.argtypes = [_i64, _i64, _i64]
    L.nvfp4_pack.restype = _i32
    L.nvfp4_pack.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]
    L.nvfp4_quantize.restype = _i32
    L.nvfp4_quantize.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
    L.nvfp4_dequant_f32.restype = _i32
    L.nvfp4_dequant_f32.argtypes = [_vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp]
    L.nvfp4_skinny_gemm.restype = _i32
    L.nvfp4_skinny_gemm.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp, _vp]
    L.fp8_skinny_gemm.restype = _i32
    L.fp8_skinny_gemm.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp]
    L.moe_route_topk.restype = _i32
    L.moe_route_topk.argtypes = [_vp, _vp, _i64, _i64, _i64] + [_vp] * 9
    L.moe_route_project_topk.restype = _i32
    L.moe_route_project_topk.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64] + [_vp] * 10
    L.moe_nvfp4_workspace_bytes.restype = _i64
    L.moe_nvfp4_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, _i32]
    L.moe_nvfp4_decode.restype = _i32
    L.moe_nvfp4_decode.argtypes = [ctypes.POINTER(MoeArgs), _vp]
    L.moe_nvfp4_route_decode.restype = _i32
    L.moe_nvfp4_route_decode.argtypes = [ctypes.POINTER(MoeArgs), _vp, _vp, _vp]
    L.moe_nvfp4_route_decode_static.restype = _i32
    L.moe_nvfp4_route_decode_static.argtypes = [ctypes.POINTER(MoeArgs), _vp, _vp, _vp]
    L.nvfp4moe_stream_blocks.restype = _i64
    L.nvfp4moe_stream_blocks.argtypes = [_i64]
    L.nvfp4moe_stream_read.restype = _i32
    L.nvfp4moe_stream_read.argtypes = [_vp, _i64, _vp, _i64, _vp]
    return L


lib = _load()

EXPORTS = ["nvfp4moe_strerror", "nvfp4moe_last_error_detail", "nvfp4moe_version",
           "fp8_skinny_gemm",
           "nvfp4_packed_bytes", "nvfp4_pack", "nvfp4_quantize", "nvfp4_dequant_f32", "nvfp4_skinny_gemm",
           "moe_route_topk", "moe_route_project_topk", "moe_nvfp4_workspace_bytes", "moe_nvfp4_decode",
           "moe_nvfp4_route_decode", "moe_nvfp4_route_decode_static", "nvfp4moe_stream_blocks",
           "nvfp4moe_stream_read"]


def strerror(status: int) -> str:
    return lib.nvfp4moe_strerror(status).decode()


def last_error_detail() -> str:
    return lib.nvfp4moe_last_error_detail().decode()


def version() -> str:
    return lib.nvfp4moe_version().decode()


def _check(status: int, where: str):
    if status != NVFP4MOE_OK:
        raise NVFP4MoEError(status, where, last_error_detail())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _want(t: Optional[torch.Tensor], name: str, shape, dtype, device):
    """Raises ValueError unless t is None or a contiguous tensor of this
    shape and dtype on `device` (the kernels index it by these sizes)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, x on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ---- weights ------------------------------------------------------------------------

@dataclass
class PackedNVFP4:
    """G packed matrices of N x K in the library layout (device bytes)."""
    data: torch.Tensor  # uint8, nvfp4_packed_bytes(G, N, K)
    G: int
    N: int
    K: int


def nvfp4_packed_bytes(G: int, N: int, K: int) -> int:
    n = lib.nvfp4_packed_bytes(G, N, K)
    if n < 0:
        raise NVFP4MoEError(int(n), "nvfp4_packed_bytes", last_error_detail())
    return int(n)


def nvfp4_pack(codes: torch.Tensor, scales: torch.Tensor, g: torch.Tensor, stream=None,
               out: Optional[torch.Tensor] = None) -> PackedNVFP4:
    """codes uint8 [G][N][K/2], scales uint8 [G][N][K/16], g float32 [G] (GPU)."""
    G, N, kh = codes.shape
    K = kh * 2
    if tuple(scales.shape) != (G, N, K // 16) or tuple(g.shape) != (G,):
        raise ValueError("scales must be [G][N][K/16] and g [G]")
    nbytes = nvfp4_packed_bytes(G, N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib.nvfp4_pack(_ptr(codes), _ptr(scales), _ptr(g), G, N, K, _ptr(out),
                          _stream(stream)), "nvfp4_pack")
    return PackedNVFP4(out, G, N, K)


def nvfp4_quantize(x: torch.Tensor, stream=None):
    """x bfloat16 [G][N][K] (or [N][K]) -> canonical NVFP4 (codes uint8
    [G][N][K/2], scales uint8 [G][N][K/16], g float32 [G]) on x's device."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    if x.dim() == 2:
        x = x.unsqueeze(0)
    x = x.contiguous()
    G, N, K = x.shape
    codes = torch.empty((G, N, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((G, N, K // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(G, dtype=torch.float32, device=x.device)
    _check(lib.nvfp4_quantize(_ptr(x), G, N, K, _ptr(codes), _ptr(scales), _ptr(g),
                              _stream(stream)), "nvfp4_quantize")
    return codes, scales, g


def nvfp4_dequant_f32(w: PackedNVFP4, apply_g: bool = True, path: int = 0,
                      stream=None) -> torch.Tensor:
    out = torch.empty((w.G, w.N, w.K), dtype=torch.float32, device=w.data.device)
    _check(lib.nvfp4_dequant_f32(_ptr(w.data), w.G, w.N, w.K, int(apply_g), int(path),
                                 _ptr(out), _stream(stream)), "nvfp4_dequant_f32")
    return out


def nvfp4moe_stream_blocks(nbytes: int) -> int:
    n = lib.nvfp4moe_stream_blocks(nbytes)
    if n < 0:
        raise NVFP4MoEError(int(n), "nvfp4moe_stream_blocks", last_error_detail())
    return int(n)


def nvfp4moe_stream_read(src: torch.Tensor, stream=None,
                         sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reads src (any dtype, contiguous, a multiple of 16 bytes) once; returns
    the sink, int32 [blocks], whose XOR is the XOR of src's 32-bit words."""
    nbytes = src.numel() * src.element_size()
    blocks = nvfp4moe_stream_blocks(nbytes)
    if sink is None:
        sink = torch.empty(blocks, dtype=torch.int32, device=src.device)
    _check(lib.nvfp4moe_stream_read(_ptr(src), nbytes, _ptr(sink), sink.numel(), _stream(stream)),
           "nvfp4moe_stream_read")
    return sink


def nvfp4_skinny_gemm(x: torch.Tensor, w: PackedNVFP4, stream=None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x bfloat16 [M][K] -> bfloat16 [M][N] = x W^T."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    M, K = x.shape
    if K != w.K or w.G != 1:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    _want(out, "out", (M, w.N), torch.bfloat16, x.device)
    _check(lib.nvfp4_skinny_gemm(_ptr(x), M, K, _ptr(w.data), w.N, _ptr(out), _stream(stream)),
           "nvfp4_skinny_gemm")
    return out


def fp8_skinny_gemm(x: torch.Tensor, w_fp8: torch.Tensor, scale: torch.Tensor, stream=None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x bfloat16 [M][K], w_fp8 uint8 [N][K] (E4M3 codes), scale float32 [1]
    -> bfloat16 [M][N] = (x W^T) * scale."""
    if x.dtype != torch.bfloat16 or w_fp8.dtype != torch.uint8 or scale.dtype != torch.float32:
        raise ValueError("need bfloat16 x, uint8 w_fp8, float32 scale")
    M, K = x.shape
    N = w_fp8.shape[0]
    if w_fp8.shape[1] != K:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _want(out, "out", (M, N), torch.bfloat16, x.device)
    _check(lib.fp8_skinny_gemm(_ptr(x), M, K, _ptr(w_fp8), _ptr(scale), N, _ptr(out),
                               _stream(stream)), "fp8_skinny_gemm")
    return out


# ---- routing -------------------------------------------------------------------------

@dataclass
class Routing:
    ids: torch.Tensor       # int32 [M][k]
    w: torch.Tensor         # float32 [M][k]
    counts: torch.Tensor    # int32 [E]
    offsets: torch.Tensor   # int32 [E+1]
    pairs: torch.Tensor     # int32 [M*k]
    active: torch.Tensor    # int32 [E]
    active_offsets: torch.Tensor  # int32 [E+1]
    n_active: torch.Tensor  # int32 [1]


def routing_buffers(M: int, E: int, k: int, device) -> Routing:
    i32 = dict(dtype=torch.int32, device=device)
    return Routing(torch.empty((M, k), **i32), torch.empty((M, k), dtype=torch.float32,
                                                           device=device),
                   torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(M * k, **i32),
                   torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(1, **i32))


def moe_route_topk(logits: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None,
                   stream=None, out: Optional[Routing] = None) -> Routing:
    """logits float32 [M][E] (+ bias float32 [E])."""
    if logits.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise ValueError("logits and bias must be float32")
    M, E = logits.shape
    r = routing_buffers(M, E, k, logits.device) if out is None else out
    _check(lib.moe_route_topk(_ptr(logits), _ptr(bias), M, E, k, _ptr(r.ids), _ptr(r.w),
                              _ptr(r.counts), _ptr(r.offsets), _ptr(r.pairs), _ptr(r.active),
                              _ptr(r.active_offsets), _ptr(r.n_active), _stream(stream)),
           "moe_route_topk")
    return r


def moe_route_project_topk(x: torch.Tensor, w_router: torch.Tensor, k: int,
                           bias: Optional[torch.Tensor] = None, stream=None,
                           out: Optional[Routing] = None,
                           logits: Optional[torch.Tensor] = None):
    """x bfloat16 [M][H], w_router bfloat16 [E][H] (+ bias float32 [E]) ->
    (logits float32 [M][E], Routing): the router projection, then top-k."""
    if x.dtype != torch.bfloat16 or w_router.dtype != torch.bfloat16:
        raise ValueError("x and w_router must be bfloat16")
    if bias is not None and bias.dtype != torch.float32:
        raise ValueError("bias must be float32")
    M, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("shape mismatch")
    r = routing_buffers(M, E, k, x.device) if out is None else out
    if logits is None:
        logits = torch.empty((M, E), dtype=torch.float32, device=x.device)
    _check(lib.moe_route_project_topk(_ptr(x), _ptr(w_router), _ptr(bias), M, E, k, H,
                                      _ptr(logits), _ptr(r.ids), _ptr(r.w), _ptr(r.counts),
                                      _ptr(r.offsets), _ptr(r.pairs), _ptr(r.active),
                                      _ptr(r.active_offsets), _ptr(r.n_active), _stream(stream)),
           "moe_route_project_topk")
    return logits, r


# ---- MoE block ---------------------------------------------------------------------------

def moe_nvfp4_workspace_bytes(M: int, E: int, k: int, H: int, I: int, has_shared: bool) -> int:
    n = lib.moe_nvfp4_workspace_bytes(M, E, k, H, I, int(has_shared))
    if n < 0:
        raise NVFP4MoEError(int(n), "moe_nvfp4_workspace_bytes", last_error_detail())
    return int(n)


def moe_workspace(M: int, E: int, k: int, H: int, I: int, has_shared: bool,
                  device) -> torch.Tensor:
    """A workspace for these sizes (needs no initialisation)."""
    return torch.empty(moe_nvfp4_workspace_bytes(M, E, k, H, I, has_shared), dtype=torch.uint8,
                       device=device)


def _check_block_args(x, E, k, H, I, residual, out, ids, w, workspace, shared_gate_up,
                      shared_down):
    M = x.shape[0]
    dev = x.device
    _want(residual, "residual", (M, H), torch.bfloat16, dev)
    _want(out, "out", (M, H), torch.bfloat16, dev)
    _want(ids, "ids", (M, k), torch.int32, dev)
    _want(w, "w", (M, k), torch.float32, dev)
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != dev
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
    if (shared_gate_up is None) != (shared_down is None):
        raise ValueError("shared_gate_up and shared_down go together")
    if shared_gate_up is not None:
        if (shared_gate_up.G, shared_gate_up.N, shared_gate_up.K) != (1, 2 * I, H) or \
                (shared_down.G, shared_down.N, shared_down.K) != (1, H, I):
            raise ValueError("shared expert shapes do not match the routed experts")


def moe_nvfp4_decode(x: torch.Tensor, routing: Routing, w_gate_up: PackedNVFP4,
                     w_down: PackedNVFP4, shared_gate_up: Optional[PackedNVFP4] = None,
                     shared_down: Optional[PackedNVFP4] = None,
                     residual: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None,
                     out: Optional[torch.Tensor] = None, schedule: int = SCHEDULE_AUTO,
                     dense_min_rows: int = 0) -> torch.Tensor:
    """x bfloat16 [M][H] -> bfloat16 [M][H] (routed experts + shared + residual).
    schedule: SCHEDULE_AUTO / SCHEDULE_THREE_LAUNCHES / SCHEDULE_TWO_LAUNCHES;
    dense_min_rows: rows from which a slot uses MFMA (0 = library default)."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    M, H = x.shape
    E, I = w_gate_up.G, w_down.K
    k = routing.ids.shape[1]
    if w_gate_up.N != 2 * I or w_gate_up.K != H or w_down.N != H or w_down.G != E:
        raise ValueError("expert weight shapes do not match x")
    _check_block_args(x, E, k, H, I, residual, out, routing.ids, routing.w, workspace,
                      shared_gate_up, shared_down)
    dev = x.device
    for name, t, n in (("offsets", routing.offsets, E + 1), ("pairs", routing.pairs, M * k),
                       ("active", routing.active, E),
                       ("active_offsets", routing.active_offsets, E + 1),
                       ("n_active", routing.n_active, 1)):
        _want(t, name, (n,), torch.int32, dev)
    has_shared = shared_gate_up is not None
    if workspace is None:
        workspace = moe_workspace(M, E, k, H, I, has_shared, x.device)
    if out is None:
        out = torch.empty_like(x)
    a = MoeArgs()
    a.x, a.ids, a.w = _ptr(x), _ptr(routing.ids), _ptr(routing.w)
    a.offsets, a.pairs = _ptr(routing.offsets), _ptr(routing.pairs)
    a.active, a.n_active = _ptr(routing.active), _ptr(routing.n_active)
    a.active_offsets = _ptr(routing.active_offsets)
    a.w_gate_up, a.w_down = _ptr(w_gate_up.data), _ptr(w_down.data)
    a.shared_gate_up = _ptr(shared_gate_up.data) if has_shared else None
    a.shared_down = _ptr(shared_down.data) if has_shared else None
    a.residual = _ptr(residual)
    a.out = _ptr(out)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    a.M, a.E, a.k, a.H, a.I = M, E, k, H, I
    a.dense_min_rows, a.schedule = dense_min_rows, schedule
    _check(lib.moe_nvfp4_decode(ctypes.byref(a), _stream(stream)), "moe_nvfp4_decode")
    return out


def moe_nvfp4_route_decode(x: torch.Tensor, logits: torch.Tensor, k: int,
                           w_gate_up: PackedNVFP4, w_down: PackedNVFP4,
                           bias: Optional[torch.Tensor] = None,
                           shared_gate_up: Optional[PackedNVFP4] = None,
                           shared_down: Optional[PackedNVFP4] = None,
                           residual: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None,
                           out: Optional[torch.Tensor] = None,
                           ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                           dense_min_rows: int = 0, proj: Optional[PackedNVFP4] = None,
                           proj_out: Optional[torch.Tensor] = None,
                           static_scratch: bool = False):
    """Routing (top-k + weights) and the MoE block in two launches, for few
    rows: x bfloat16 [M][H], logits float32 [M][E] (+ bias float32 [E]) ->
    (out bfloat16 [M][H], ids int32 [M][k], w float32 [M][k]). With proj
    (packed [N][H]), proj_out bfloat16 [M][N] = x proj^T is written too, by
    blocks of the down launch (allocated if not given).
    static_scratch: call moe_nvfp4_route_decode_static, whose h rows live in
    the library's own device array (no workspace; pass out, ids and w to
    allocate nothing here either)."""
    if x.dtype != torch.bfloat16 or logits.dtype != torch.float32:
        raise ValueError("x must be bfloat16 and logits float32")
    if bias is not None and bias.dtype != torch.float32:
        raise ValueError("bias must be float32")
    M, H = x.shape
    E, I = w_gate_up.G, w_down.K
    if w_gate_up.N != 2 * I or w_gate_up.K != H or w_down.N != H or w_down.G != E:
        raise ValueError("expert weight shapes do not match x")
    if tuple(logits.shape) != (M, E):
        raise ValueError("logits must be [M][E]")
    _want(logits, "logits", (M, E), torch.float32, x.device)
    _want(bias, "bias", (E,), torch.float32, x.device)
    _check_block_args(x, E, k, H, I, residual, out, ids, w, workspace, shared_gate_up,
                      shared_down)
    has_shared = shared_gate_up is not None
    if workspace is None and not static_scratch:
        workspace = moe_workspace(M, E, k, H, I, has_shared, x.device)
    if out is None:
        out = torch.empty_like(x)
    if ids is None:
        ids = torch.empty((M, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=x.device)
    a = MoeArgs()
    a.x, a.ids, a.w = _ptr(x), _ptr(ids), _ptr(w)
    a.w_gate_up, a.w_down = _ptr(w_gate_up.data), _ptr(w_down.data)
    a.shared_gate_up = _ptr(shared_gate_up.data) if has_shared else None
    a.shared_down = _ptr(shared_down.data) if has_shared else None
    a.residual = _ptr(residual)
    a.out = _ptr(out)
    if not static_scratch:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    a.M, a.E, a.k, a.H, a.I = M, E, k, H, I
    a.dense_min_rows, a.schedule = dense_min_rows, SCHEDULE_AUTO
    if proj is not None:
        if proj.G != 1 or proj.K != H:
            raise ValueError("proj must be one packed [N][H] matrix")
        if proj_out is None:
            proj_out = torch.empty((M, proj.N), dtype=torch.bfloat16, device=x.device)
        _want(proj_out, "proj_out", (M, proj.N), torch.bfloat16, x.device)
        a.proj_w, a.proj_n, a.proj_out = _ptr(proj.data), proj.N, _ptr(proj_out)
    if static_scratch:
        _check(lib.moe_nvfp4_route_decode_static(ctypes.byref(a), _ptr(logits), _ptr(bias),
                                                 _stream(stream)), "moe_nvfp4_route_decode_static")
    else:
        _check(lib.moe_nvfp4_route_decode(ctypes.byref(a), _ptr(logits), _ptr(bias),
                                          _stream(stream)), "moe_nvfp4_route_decode")
    return out, ids, w
