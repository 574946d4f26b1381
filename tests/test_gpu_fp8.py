"""GPU parity of the FP8 E4M3 skinny product (one FP32 scale per tensor, the
attention-projection product of the Elsa page, "An FP8 fast path") against the
oracle, through the C ABI: decode bit for bit, sums under
|gpu - ref| <= 1e-2 |ref| + 1e-3 against the oracle's float64 result."""
import numpy as np
import pytest
import torch

import oracle
from synth.workloads import fp8_projection
from tests.helpers import dev_bf16_to_f64, to_dev_bf16, tol_ratio

pytestmark = pytest.mark.gpu

FINITE_E4M3 = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)


@pytest.fixture(scope="module")
def m(gpu):
    import nvfp4_moe_skinny_amd as m
    return m


def _run(m, gpu, x, w, s):
    sc = torch.tensor([s], dtype=torch.float32, device=gpu)
    y = m.fp8_skinny_gemm(to_dev_bf16(x, gpu), torch.from_numpy(w).to(gpu), sc)
    torch.cuda.synchronize()
    return dev_bf16_to_f64(y)


@pytest.mark.parametrize("M,K,N", [(1, 2048, 5120), (4, 2048, 5120), (8, 4096, 2048),
                                   (16, 2048, 512), (3, 1024, 100), (5, 1024, 8 * 13 + 3),
                                   (7, 4096, 3), (2, 2048, 1), (13, 1024, 4097)])
def test_fp8_gemm_parity(m, gpu, M, K, N):
    """Full tiles and ragged tails (N not a multiple of the rows per tile),
    row counts across and between batches of four."""
    x, w, s = fp8_projection(seed=M + N, M=M, K=K, N=N)
    got = _run(m, gpu, x, w, s)
    ref = oracle.gemm_fp8(x, w, s)
    assert np.isfinite(got).all()
    assert tol_ratio(got, ref) <= 1.0


@pytest.mark.parametrize("K", [1024, 2048, 4096])
@pytest.mark.parametrize("s", [1.0, 2.0 ** -9])
def test_fp8_decode_bit_exact_every_code(m, gpu, K, s):
    """Unit rows of x read single weights back: every finite E4M3 code (incl.
    subnormals and -0) times a power-of-two scale is a BF16 value, so each
    output must equal the oracle's exactly."""
    cols = [0, 15, 16, K // 2 + 9, K - 1]
    x = np.zeros((len(cols), K), np.uint16)
    for r, c in enumerate(cols):
        x[r, c] = 0x3F80  # 1.0
    rng = np.random.default_rng(K)
    N = len(FINITE_E4M3) * 2 + 5
    w = rng.choice(FINITE_E4M3, (N, K)).astype(np.uint8)
    for r, c in enumerate(cols):
        w[:, c] = np.resize(np.roll(FINITE_E4M3, 37 * r), N)
    got = _run(m, gpu, x, w, s)
    ref = oracle.gemm_fp8(x, w, s)
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    assert (ref_bf16 == ref).all()  # the expected values are BF16 values
    assert (got == ref).all()
    # -0 (0x80) reads back as zero
    assert (got[w[:, cols].T == 0x80] == 0).all()


def test_fp8_gemm_repeat_and_out_buffer(m, gpu):
    """Same inputs, same bits (fixed summation order); a caller's output
    buffer and a second stream give the same result."""
    x, w, s = fp8_projection(seed=3, M=4, K=2048, N=640)
    xd, wd = to_dev_bf16(x, gpu), torch.from_numpy(w).to(gpu)
    sc = torch.tensor([s], dtype=torch.float32, device=gpu)
    a = m.fp8_skinny_gemm(xd, wd, sc)
    st = torch.cuda.Stream()
    out = torch.full((4, 640), float("nan"), dtype=torch.bfloat16, device=gpu)
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        b = m.fp8_skinny_gemm(xd, wd, sc, stream=st, out=out)
    st.synchronize()
    torch.cuda.synchronize()
    assert b.data_ptr() == out.data_ptr()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
