"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, and rejects bad arguments with the
documented status codes before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


@pytest.fixture(scope="module")
def m():
    import nvfp4_moe_skinny_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(m):
    names = declared_functions()
    assert set(m.EXPORTS) == set(names), names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(m):
    for code, name in [(0, "NVFP4MOE_OK"), (-1, "NVFP4MOE_ERR_NULL_ARG"),
                       (-2, "NVFP4MOE_ERR_BAD_SHAPE"), (-3, "NVFP4MOE_ERR_UNSUPPORTED"),
                       (-4, "NVFP4MOE_ERR_WORKSPACE"), (-5, "NVFP4MOE_ERR_HIP")]:
        assert m.strerror(code) == name
    assert m.strerror(7) == "NVFP4MOE_ERR_UNKNOWN"
    assert "gfx950" in m.version()


def test_packed_bytes(m):
    # tile = 8 KB codes + 1 KB scales; 16384 / K rows per tile
    assert m.nvfp4_packed_bytes(1, 512, 2048) == 64 * 9216 + 256
    assert m.nvfp4_packed_bytes(256, 1024, 2048) == 256 * 128 * 9216 + 1024
    assert m.nvfp4_packed_bytes(256, 2048, 512) == 256 * 64 * 9216 + 1024
    assert m.nvfp4_packed_bytes(1, 33, 512) == 2 * 9216 + 256     # ragged rows pad
    # K % 32 == 0 in general: Q = K / Kp panels of Kp = the largest 32 * 2^j <= 2048
    # dividing K; a row block is Q tiles of 16384 / Kp rows
    assert m.nvfp4_packed_bytes(1, 600, 96) == 2 * 3 * 9216 + 256      # Kp 32: 512 rows
    assert m.nvfp4_packed_bytes(1, 512, 1536) == 16 * 3 * 9216 + 256   # Kp 512: 32 rows
    assert m.nvfp4_packed_bytes(1, 17, 3072) == 2 * 3 * 9216 + 256     # Kp 1024: 16 rows
    assert m.nvfp4_packed_bytes(2, 2048, 4096) == 2 * 256 * 2 * 9216 + 256  # Kp 2048
    assert m.nvfp4_packed_bytes(1, 8, 65536) == 32 * 9216 + 256
    for K in (16, 48, 100, 65568, 0):
        assert m.lib.nvfp4_packed_bytes(1, 8, K) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert m.lib.nvfp4_packed_bytes(0, 8, 64) == m.NVFP4MOE_ERR_BAD_SHAPE


def test_validation_errors_before_launch(m):
    L = m.lib
    fake = 4096  # never dereferenced: every call below fails validation first
    assert L.nvfp4_pack(None, fake, fake, 1, 8, 64, fake, None) == m.NVFP4MOE_ERR_NULL_ARG
    assert L.nvfp4_pack(fake, fake, fake, 1, 8, 80 + 8, fake, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.nvfp4_dequant_f32(fake, 1, 8, 64, 1, 2, fake, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.nvfp4_skinny_gemm(fake, 0, 64, fake, 8, fake, None) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.nvfp4_skinny_gemm(fake, 1, 4100, fake, 8, fake, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.nvfp4_skinny_gemm(fake, 1, 1 << 17, fake, 8, fake, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.nvfp4_skinny_gemm(fake + 2, 1, 64, fake, 8, fake, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # misaligned x
    assert L.fp8_skinny_gemm(None, 1, 2048, fake, fake, 8, fake, None) == m.NVFP4MOE_ERR_NULL_ARG
    assert L.fp8_skinny_gemm(fake, 0, 2048, fake, fake, 8, fake, None) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.fp8_skinny_gemm(fake, 1, 2048, fake, fake, 0, fake, None) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.fp8_skinny_gemm(fake, 1, 512, fake, fake, 8, fake, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # K not 1024, 2048 or 4096
    assert L.fp8_skinny_gemm(fake, 1, 2048, fake + 8, fake, 8, fake, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # misaligned weights
    r = [fake] * 8
    assert L.moe_route_topk(None, None, 4, 256, 8, *r, None) == m.NVFP4MOE_ERR_NULL_ARG
    assert L.moe_route_topk(fake, None, 4, 257, 8, *r, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.moe_route_topk(fake, None, 4, 256, 9, *r, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.moe_route_topk(fake, None, 4, 4, 5, *r, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.moe_route_topk(fake, None, 0, 256, 8, *r, None) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.moe_route_topk(fake, None, 2000, 256, 8, *r, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert "k" in m.last_error_detail() or "M" in m.last_error_detail()
    assert L.nvfp4_quantize(None, 1, 8, 32, fake, fake, fake, None) == m.NVFP4MOE_ERR_NULL_ARG
    assert L.nvfp4_quantize(fake, 0, 8, 32, fake, fake, fake, None) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.nvfp4_quantize(fake, 1, 8, 40, fake, fake, fake, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # K % 16
    assert L.nvfp4_quantize(fake + 8, 1, 8, 32, fake, fake, fake, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # misaligned x
    rp = [fake] * 9
    assert L.moe_route_project_topk(None, fake, None, 4, 256, 8, 2048, fake, *rp, None) == \
        m.NVFP4MOE_ERR_NULL_ARG
    assert L.moe_route_project_topk(fake, fake, None, 4, 256, 8, 2048, None, *rp, None) == \
        m.NVFP4MOE_ERR_NULL_ARG  # logits buffer
    assert L.moe_route_project_topk(fake, fake, None, 0, 256, 8, 2048, fake, *rp, None) == \
        m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.moe_route_project_topk(fake, fake, None, 4, 256, 8, 256, fake, *rp, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # H
    assert L.moe_route_project_topk(fake, fake, None, 4, 257, 8, 2048, fake, *rp, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # E
    assert L.moe_route_project_topk(fake + 4, fake, None, 4, 256, 8, 2048, fake, *rp, None) == \
        m.NVFP4MOE_ERR_UNSUPPORTED  # misaligned x


def test_stream_read_validation(m):
    L = m.lib
    fake = 4096
    # 1 vector per thread below 512 MiB, 8 from there on; at most 8192 workgroups
    assert m.nvfp4moe_stream_blocks(16) == 1
    assert m.nvfp4moe_stream_blocks(256 * 16) == 1
    assert m.nvfp4moe_stream_blocks(256 * 16 + 16) == 2
    assert m.nvfp4moe_stream_blocks(512 << 20) == 8192
    assert m.nvfp4moe_stream_blocks(1 << 34) == 8192  # capped: the grid strides beyond
    assert L.nvfp4moe_stream_blocks(15) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.nvfp4moe_stream_read(None, 64, fake, 1, None) == m.NVFP4MOE_ERR_NULL_ARG
    assert L.nvfp4moe_stream_read(fake, 0, fake, 1, None) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert L.nvfp4moe_stream_read(fake, 40, fake, 1, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.nvfp4moe_stream_read(fake + 4, 64, fake, 1, None) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert L.nvfp4moe_stream_read(fake, 1 << 20, fake, 1, None) == m.NVFP4MOE_ERR_WORKSPACE


def _args(m, **kw):
    a = m.MoeArgs()
    fake = 4096
    for f in ("x", "ids", "w", "offsets", "pairs", "active", "active_offsets", "n_active",
              "w_gate_up", "w_down", "out", "workspace"):
        setattr(a, f, fake)
    a.workspace_bytes = 1 << 30
    a.M, a.E, a.k, a.H, a.I = 4, 256, 8, 2048, 512
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_validation(m):
    L = m.lib
    dec = lambda a: L.moe_nvfp4_decode(ctypes.byref(a), None)
    assert L.moe_nvfp4_decode(None, None) == m.NVFP4MOE_ERR_NULL_ARG
    assert dec(_args(m, x=None)) == m.NVFP4MOE_ERR_NULL_ARG
    assert dec(_args(m, shared_gate_up=4096)) == m.NVFP4MOE_ERR_NULL_ARG  # down missing
    assert dec(_args(m, M=0)) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert dec(_args(m, E=300)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert dec(_args(m, k=9)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert dec(_args(m, H=3000)) == m.NVFP4MOE_ERR_UNSUPPORTED  # not a multiple of 32
    assert dec(_args(m, I=100)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert dec(_args(m, H=2048, I=4)) == m.NVFP4MOE_ERR_UNSUPPORTED
    # the up half of gate_up must start on a row block: I % (16384 / panel_k(H)) == 0
    assert dec(_args(m, H=96, I=256)) == m.NVFP4MOE_ERR_UNSUPPORTED  # 512-row blocks
    assert "row block" in m.last_error_detail()
    assert dec(_args(m, H=1536, I=48)) == m.NVFP4MOE_ERR_UNSUPPORTED  # 32-row blocks
    assert dec(_args(m, H=1 << 17)) == m.NVFP4MOE_ERR_UNSUPPORTED
    need = m.moe_nvfp4_workspace_bytes(4, 256, 8, 2048, 512, False)
    assert dec(_args(m, workspace_bytes=need - 1)) == m.NVFP4MOE_ERR_WORKSPACE
    assert "workspace" in m.last_error_detail()
    assert dec(_args(m, x=4096 + 8)) == m.NVFP4MOE_ERR_UNSUPPORTED  # misaligned
    assert dec(_args(m, schedule=4)) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert dec(_args(m, schedule=1)) == m.NVFP4MOE_ERR_BAD_SHAPE
    # (M*k + M) items x 256 tiles of a 2048 x 2048 matrix would pass 2^31 blocks
    assert dec(_args(m, M=1_000_000, I=2048)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert "grid" in m.last_error_detail()
    # two launches need FP32 h for every pair: no MFMA slot (M < dense_min_rows)
    assert dec(_args(m, schedule=3, dense_min_rows=4)) == m.NVFP4MOE_ERR_UNSUPPORTED
    # the library's default threshold for 9 <= M <= 16 is 3 rows (MFMA slots)
    assert dec(_args(m, M=12, schedule=3)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert dec(_args(m, ids=None)) == m.NVFP4MOE_ERR_NULL_ARG
    # routing folded in: grouping arrays not needed; logits required; M < dense_min_rows
    rd = lambda a, lg=4096: L.moe_nvfp4_route_decode(ctypes.byref(a), lg, None, None)
    assert rd(_args(m), lg=None) == m.NVFP4MOE_ERR_NULL_ARG
    assert rd(_args(m, w=None)) == m.NVFP4MOE_ERR_NULL_ARG
    assert rd(_args(m, M=16)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert rd(_args(m, M=4, dense_min_rows=3)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert rd(_args(m, workspace_bytes=1)) == m.NVFP4MOE_ERR_WORKSPACE
    assert dec(_args(m, schedule=-1)) == m.NVFP4MOE_ERR_BAD_SHAPE
    # the projection rides on moe_nvfp4_route_decode only, within its limits
    pj = dict(proj_w=4096, proj_n=64, proj_out=4096)
    assert dec(_args(m, **pj)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert rd(_args(m, proj_w=4096, proj_n=64)) == m.NVFP4MOE_ERR_NULL_ARG
    assert rd(_args(m, proj_w=4096, proj_n=0, proj_out=4096)) == m.NVFP4MOE_ERR_BAD_SHAPE
    assert rd(_args(m, proj_w=4096, proj_n=4097, proj_out=4096)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert rd(_args(m, k=2, **pj)) == m.NVFP4MOE_ERR_UNSUPPORTED  # fewer than 4 waves
    assert rd(_args(m, H=1024, **pj)) == m.NVFP4MOE_ERR_UNSUPPORTED
    assert rd(_args(m, proj_w=4096 + 8, proj_n=64, proj_out=4096)) == m.NVFP4MOE_ERR_UNSUPPORTED
    # with a projection, out and proj_out must not overlap x (4 x 2048 BF16 = 16 KB)
    big = 1 << 24
    assert rd(_args(m, x=big, out=big, **dict(pj, proj_out=2 * big))) == \
        m.NVFP4MOE_ERR_BAD_SHAPE
    assert rd(_args(m, x=big, out=big + 16384 - 16, **dict(pj, proj_out=2 * big))) == \
        m.NVFP4MOE_ERR_BAD_SHAPE
    assert rd(_args(m, x=big, out=2 * big, **dict(pj, proj_out=big + 512))) == \
        m.NVFP4MOE_ERR_BAD_SHAPE
    assert "overlap" in m.last_error_detail()
    # h [M*k][I] and y [M*k][H] as 4-byte words
    assert need == 4 * 8 * (512 + 2048) * 4
    assert m.moe_nvfp4_workspace_bytes(4, 256, 8, 2048, 512, True) == (4 * 8 + 4) * (512 + 2048) * 4
