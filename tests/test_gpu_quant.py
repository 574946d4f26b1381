"""GPU parity of the device quantizer (BF16 -> canonical NVFP4, amax recipe)
against the oracle, through the C ABI: codes, scales and tensor scales bit
for bit (both sides take every rounding decision in FP32)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import dev_bf16_to_f64, to_dev_bf16, tol_ratio

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(gpu):
    import nvfp4_moe_skinny_amd as m
    return m


def _quant(m, gpu, x):
    c, s, g = m.nvfp4_quantize(to_dev_bf16(x, gpu))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy()


def _check(m, gpu, x, sample=None):
    c, s, g = _quant(m, gpu, x)
    idx = range(x.shape[0]) if sample is None else sample
    for i in idx:
        rc, rs, rg = oracle.quantize_nvfp4(x[i])
        assert g[i].view(np.uint32) == rg[0].view(np.uint32), i
        assert (s[i] == rs[0]).all(), i
        assert (c[i] == rc[0]).all(), i


def _bf16(v):
    return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy() \
        .astype(np.uint16)


@pytest.mark.parametrize("G,N,K,std", [(1, 4, 32, 1.0), (3, 17, 256, 1.0), (2, 64, 2048, 0.02),
                                       (4, 5, 48, 1000.0), (2, 33, 512, 1e-30),
                                       (1, 512, 1024, 1.0),
                                       (700, 2, 64, 1.0)])  # many matrices: the grid's rows
def test_quantize_bit_exact(m, gpu, G, N, K, std):
    x = synth.normal_bf16(synth.key(G, 120, N, K), (G, N, K), 0.0, std)
    # outliers, an all-zero block and negative zeros
    x[0, 0, 5] = _bf16(40.0 * std)
    if N > 1:
        x[0, 1, :16] = 0
        x[0, 1, 3] = 0x8000
    _check(m, gpu, x)


def test_quantize_zero_matrix_and_ties(m, gpu):
    K = 64
    x = np.zeros((3, 2, K), np.uint16)
    # matrix 1: g = 1 (amax 2688); block 1 scale 1.0 (t = 1); its elements on
    # every E2M1 midpoint, each side of it and on the grid
    x[1, 0, 0] = _bf16(2688.0)
    x[1, 0, 16] = _bf16(6.0)
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.5, 3.0, 6.0, -0.75, -2.5, -5.0, 4.0]
    x[1, 0, 17:17 + len(vals)] = _bf16(vals)
    nb = np.array([0.2578125, 0.7421875, 1.2578125, 1.7421875, 2.515625, 3.484375, 4.96875])
    x[1, 1, 16:16 + len(nb)] = _bf16(nb)
    x[1, 1, 0] = _bf16(6.0 * 1.0625)  # t = 1.0625, an E4M3 tie: scale 1.0, 6.375 saturates
    # matrix 2: subnormal block scales (t below 2^-6)
    x[2, 0, 0] = _bf16(2688.0)
    x[2, 0, 16:20] = _bf16([6.0 * 2.0 ** -9, 1e-3, 3e-3, -4e-4])
    x[2, 1, 0:3] = _bf16([6.0 * 1.5 * 2.0 ** -9, 6.0 * 2.0 ** -10, 6.0 * 2.5 * 2.0 ** -9])
    _check(m, gpu, x)
    c, s, g = _quant(m, gpu, x)
    assert g[0] == 1.0 and (s[0] == 0).all() and (c[0] == 0).all()


def _bf16_next(bits, up):
    """The BF16 neighbour of non-negative BF16 bit patterns, away from or toward zero."""
    return (bits.astype(np.int32) + (1 if up else -1)).astype(np.uint16)


@pytest.mark.parametrize("k", [-110, -30, 0, 25])
def test_quantize_quotients_on_midpoints(m, gpu, k):
    """Tensor scale g = 2^k (matrix amax 2688 * 2^k), every non-zero E4M3 block
    scale code s_b (block amax 6 s_b g), and elements exactly on each E2M1
    midpoint times s_b g (quotients that are exact ties) and one BF16 step to
    either side: the per-element quotients |x| / (s_b g) must be the correctly
    rounded ones for every code to match. k = -110 puts s_b g below 2^-100."""
    K = 256
    codes = np.arange(1, 0x7F)  # 126 block scales
    nblk = K // 16
    N = (len(codes) + 1 + nblk - 1) // nblk
    g = np.float32(2.0 ** k)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x = np.zeros((1, N, K), np.float32)
    x[0, 0, 0] = 2688.0 * g  # sets amax: g = 2^k exactly; block 0 scale 448
    for i, c in enumerate(codes):
        b = i + 1
        n, col = b // nblk, 16 * (b % nblk)
        s_b = float(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn)
                    .to(torch.float32)[0])
        sg = np.float32(s_b) * g
        x[0, n, col] = 6.0 * sg                       # block amax: t = s_b exactly
        x[0, n, col + 1:col + 8] = mids * sg           # exact ties
        x[0, n, col + 8:col + 15] = -mids * sg
    bits = _bf16(x.ravel().tolist()).reshape(x.shape)
    # one BF16 step away from the ties on every other block, toward zero on the rest
    for b in range(1, len(codes) + 1):
        n, col = b // nblk, 16 * (b % nblk)
        seg = bits[0, n, col + 1:col + 15]
        mag = seg & 0x7FFF
        step = _bf16_next(mag, up=(b % 2 == 0))
        seg[:] = (seg & 0x8000) | np.where(b % 3 == 0, mag, step)
        if b % 2:
            bits[0, n, col + 15] = 0x8000  # -0 inside a block with a scale: code 8
    _check(m, gpu, bits)


def test_quantize_inverts_exact_dequant(m, gpu):
    """x = dequant(c, s, g) exactly in BF16 with every block reaching 6 s_b g:
    quantizing it gives c, s, g back."""
    rng = np.random.default_rng(5)
    G, N, K = 3, 40, 256
    codes = rng.integers(0, 16, (G, N, K))
    blocks = codes.reshape(G, N, K // 16, 16)
    blocks[..., 0] = 7 | (rng.integers(0, 2, blocks.shape[:-1]) << 3)
    codes = blocks.reshape(G, N, K)
    scales = rng.integers(1, 0x7F, (G, N, K // 16)).astype(np.uint8)
    scales[:, 0, 0] = 0x7E
    g = np.array([1.0, 2.0 ** -9, 2.0 ** 3], np.float32)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    x = oracle.dequant(packed, scales, g)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c, s, gg = _quant(m, gpu, bits)
    assert (gg == g).all() and (s == scales).all() and (c == packed).all()


def test_quantize_expert_set_sampled(m, gpu):
    """32 gate_up-shaped matrices [1024][2048] in one call; matrices are
    quantized independently, three of them checked against the oracle."""
    x = synth.normal_bf16(synth.key(7, 121), (32, 1024, 2048), 0.0, 0.02)
    _check(m, gpu, x, sample=[0, 17, 31])


def test_quantize_then_product(m, gpu):
    """Device-quantized weights, packed, through the skinny product: the
    same result as the oracle's product with the oracle-quantized weights."""
    N, K, M = 300, 2048, 4
    w = synth.normal_bf16(synth.key(8, 122), (N, K), 0.0, 0.05)
    x = synth.normal_bf16(synth.key(8, 123), (M, K))
    c, s, g = m.nvfp4_quantize(to_dev_bf16(w, gpu))
    pw = m.nvfp4_pack(c, s, g)
    y = m.nvfp4_skinny_gemm(to_dev_bf16(x, gpu), pw)
    torch.cuda.synchronize()
    rc, rs, rg = oracle.quantize_nvfp4(w)
    ref = oracle.gemm(x, rc[0], rs[0], float(rg[0]))
    assert tol_ratio(dev_bf16_to_f64(y), ref) <= 1.0
