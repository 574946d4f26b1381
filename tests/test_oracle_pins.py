"""Pins of the float64 oracle against what the formats and mathematics fix.

Each test pins the oracle to something other than itself: published value
tables (tests/golden), torch's independent float8_e4m3fn decoder, exact
rational arithmetic, closed forms of constructed special cases, high-precision
decimal brute force, and invariants. CPU only.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import NVFP4, MoELayer, moe_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


# ---- independent decoders used by the pins ------------------------------------

E2M1_TABLE = {c: v for c, v in _golden("e2m1_values.txt")}


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    """torch's own float8_e4m3fn decode: a library routine independent of the oracle."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[.., K/2] bytes -> [.., K] codes, element 2b = low nibble of byte b."""
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def table_e2m1(c: np.ndarray) -> np.ndarray:
    lut = np.array([E2M1_TABLE[i] for i in range(16)], dtype=np.float64)
    lut[8] = -0.0
    return lut[c]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


FINITE_E4M3 = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)


# ---- format decode ---------------------------------------------------------------

def test_e2m1_all_codes_match_published_table():
    for c in range(16):
        v = oracle.e2m1(c)
        assert v == E2M1_TABLE[c], c
    assert math.copysign(1.0, oracle.e2m1(8)) == -1.0  # code 8 is -0
    assert math.copysign(1.0, oracle.e2m1(0)) == 1.0


def test_e4m3_all_codes_match_torch_and_anchors():
    ref = torch_e4m3(np.arange(256, dtype=np.uint8))
    for b in range(256):
        v = oracle.e4m3(b)
        if np.isnan(ref[b]):
            assert math.isnan(v), hex(b)
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), hex(b)
    for b, val in _golden("e4m3_anchors.txt"):
        v = oracle.e4m3(b)
        if math.isnan(val):
            assert math.isnan(v)
        else:
            assert v == val and math.copysign(1, v) == math.copysign(1, val), hex(b)
    finite = [b for b in range(256) if not math.isnan(oracle.e4m3(b))]
    assert len(finite) == 254
    # strictly increasing over the non-negative codes, symmetric in the sign bit
    pos = [oracle.e4m3(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))
    assert all(oracle.e4m3(b | 0x80) == -oracle.e4m3(b) for b in range(1, 0x7F))


def test_code_times_scale_is_exact_in_fp32_and_bf16():
    """Every E2M1 x finite-E4M3 product has at most 6 significant bits, so it is
    exact in FP32 and in BF16: decoding to either loses nothing."""
    v = table_e2m1(np.arange(16))
    s = torch_e4m3(FINITE_E4M3)
    prod = np.outer(v, s)
    assert (prod.astype(np.float32).astype(np.float64) == prod).all()
    bf = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert (bf == prod).all()
    for i in range(16):
        for j, b in enumerate(FINITE_E4M3):
            assert oracle.e2m1(i) * oracle.e4m3(int(b)) == prod[i, j]


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = bf16_to_f64(bits)
    got = np.array([oracle.bf16(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("g", [1.0, 0.37, 2.0 ** -9])
def test_dequant_matches_independent_decode(g):
    """Dequant (float64 and FP32) against nibble unpacking + published E2M1 table
    + torch's E4M3 decoder; every finite scale code and every element code
    appears."""
    G, N, K = 3, 16, 128
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    scales = rng.choice(FINITE_E4M3, (G, N, K // 16)).astype(np.uint8)
    scales.reshape(-1)[: len(FINITE_E4M3)] = FINITE_E4M3
    gv = np.array([g, g * 2, g / 4], dtype=np.float32)
    v = table_e2m1(unpack_nibbles(codes))
    s = np.repeat(torch_e4m3(scales), 16, axis=-1)
    ref64 = v * s * gv.astype(np.float64)[:, None, None]
    assert (oracle.dequant(codes, scales, gv) == ref64).all()
    ref32 = ((v * s).astype(np.float32) * gv[:, None, None]).astype(np.float32)
    got32 = oracle.dequant_f32(codes, scales, gv)
    assert (got32.view(np.uint32) == ref32.view(np.uint32)).all()


# ---- skinny product: exact rational brute force -------------------------------------

def _bf16_bits_in_range(rng, shape):
    """BF16 values with |x| in [2^-8, 2^8) or 0: x * 2^15 is an integer < 2^24."""
    e = rng.integers(-8, 8, shape)
    m = rng.integers(0, 128, shape)
    sign = rng.integers(0, 2, shape)
    bits = (sign << 15) | ((e + 127) << 7) | m
    bits = np.where(rng.random(shape) < 0.1, 0, bits)
    return bits.astype(np.uint16)


@pytest.mark.parametrize("M,K,N,gexp", [(1, 16, 1, 0), (2, 32, 5, -9), (3, 64, 8, 3),
                                        (3, 64, 7, -8)])
def test_gemm_equals_exact_rational_sum(M, K, N, gexp):
    """Inside this range every product and partial sum is a dyadic rational
    that float64 holds exactly, so the oracle must equal the exact sum bit for
    bit (codes from all 16, scales from all 254 finite codes incl. subnormal
    and negative)."""
    rng = np.random.default_rng(M * 1000 + K + N)
    x = _bf16_bits_in_range(rng, (M, K))
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.choice(FINITE_E4M3, (N, K // 16)).astype(np.uint8)
    g = 2.0 ** gexp
    xf = [[Fraction(float(v)) for v in row] for row in bf16_to_f64(x)]
    cu = unpack_nibbles(codes)
    sv = torch_e4m3(scales)
    got = oracle.gemm(x, codes, scales, g)
    for m in range(M):
        for n in range(N):
            exact = sum(xf[m][k] * Fraction(E2M1_TABLE[int(cu[n, k])]) *
                        Fraction(float(sv[n, k // 16])) for k in range(K)) * Fraction(g)
            assert got[m, n] == float(exact) and Fraction(got[m, n]) == exact, (m, n)


def test_gemm_special_cases():
    rng = np.random.default_rng(11)
    M, K, N = 2, 64, 4
    x = synth.normal_bf16(synth.key(1), (M, K))
    xd = bf16_to_f64(x)
    # one non-zero weight: y = x_k * w
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    codes[1, 37 // 2] = 5 << 4          # element 37 (odd -> high nibble) = 3.0
    scales[1, 37 // 16] = 0x2B          # 2^-2 * 1.375
    y = oracle.gemm(x, codes, scales, 0.5)
    assert (y[:, [0, 2, 3]] == 0).all()
    assert (y[:, 1] == xd[:, 37] * 3.0 * 0.34375 * 0.5).all()
    # all codes c, all scales 1.0: y = e2m1(c) * g * sum(x)
    for c in range(16):
        codes = np.full((N, K // 2), c | (c << 4), np.uint8)
        scales = np.full((N, K // 16), 0x38, np.uint8)
        y = oracle.gemm(x, codes, scales, 0.25)
        ref = E2M1_TABLE[c] * 0.25 * np.array([math.fsum(r) for r in xd])
        assert np.allclose(y, ref[:, None], rtol=1e-15, atol=1e-15)
    # doubling g doubles y exactly
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.choice(FINITE_E4M3, (N, K // 16)).astype(np.uint8)
    assert (oracle.gemm(x, codes, scales, 0.75) * 2 == oracle.gemm(x, codes, scales, 1.5)).all()


# ---- quantization BF16 -> NVFP4 (amax recipe) --------------------------------------------

def _f32(v):
    return float(np.float32(v))


def test_e4m3_rne_matches_torch():
    """The oracle's nearest-code search against torch's own float32 ->
    float8_e4m3fn conversion (round to nearest even) on every E4M3 value, every
    midpoint between neighbours and the floats just either side of each."""
    vals = sorted({oracle.e4m3(c) for c in range(0x7F)})
    ts = set(vals)
    for a, b in zip(vals, vals[1:]):
        mid = np.float32((a + b) / 2)
        ts.update([float(mid), float(np.nextafter(mid, np.float32(0))),
                   float(np.nextafter(mid, np.float32(1e9)))])
    rng = np.random.default_rng(3)
    ts.update(float(v) for v in (2.0 ** rng.uniform(-12, 8.8, 2000)).astype(np.float32))
    ts = np.array(sorted(t for t in ts if t <= 448.0), np.float32)
    ref = torch.from_numpy(ts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_rne(float(t)) for t in ts], np.uint8)
    assert (got == ref).all()
    assert oracle.e4m3_rne(449.0) == 0x7E and oracle.e4m3_rne(1e30) == 0x7E  # saturates


def test_e2m1_rne_closed_form():
    """Thresholds of round-to-nearest-even on {0, .5, 1, 1.5, 2, 3, 4, 6}:
    midpoints go to the even code, everything above 5 to 6."""
    table = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for mid, code in table:
        assert oracle.e2m1_rne(mid) == code, mid
        lo, hi = np.nextafter(np.float32(mid), np.float32(0)), np.nextafter(np.float32(mid),
                                                                             np.float32(9))
        below = [c for c in range(8) if E2M1_TABLE[c] < mid][-1]
        above = [c for c in range(8) if E2M1_TABLE[c] > mid][0]
        assert oracle.e2m1_rne(float(lo)) == below and oracle.e2m1_rne(float(hi)) == above
    for c in range(8):
        assert oracle.e2m1_rne(E2M1_TABLE[c]) == c
    assert oracle.e2m1_rne(6.5) == 7 and oracle.e2m1_rne(1e30) == 7


def _nvfp4_with_full_blocks(rng, G, N, K, gexp):
    """Codes with a +-6 in every 16-block, every finite positive scale code
    in use, one 448 scale per matrix, g = 2^gexp: every value is a BF16 value
    and each block's amax is exactly 6 s_b g."""
    codes = rng.integers(0, 16, (G, N, K))
    blocks = codes.reshape(G, N, K // 16, 16)
    pos = rng.integers(0, 16, (G, N, K // 16))
    np.put_along_axis(blocks, pos[..., None], (7 | (rng.integers(0, 2, pos.shape) << 3))[..., None],
                      axis=-1)
    codes = blocks.reshape(G, N, K)
    scales = rng.integers(1, 0x7F, (G, N, K // 16)).astype(np.uint8)
    scales[:, 0, 0] = 0x7E
    g = np.full(G, 2.0 ** gexp, np.float32)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scales, g


@pytest.mark.parametrize("G,N,K,gexp", [(1, 4, 32, 0), (2, 3, 64, -12), (3, 5, 128, -7)])
def test_quantize_inverts_exact_dequant(G, N, K, gexp):
    """x = dequant(c, s, g) is exact in BF16 and its blocks meet the recipe's
    fixed point (g = amax / 2688, s_b = amax_b / 6g, q = x / s_b g exactly),
    so quantizing x must give back c, s and g bit for bit (a wrong nibble
    order, block index or sign shows)."""
    rng = np.random.default_rng(G * 100 + N + K)
    codes, scales, g = _nvfp4_with_full_blocks(rng, G, N, K, gexp)
    x = oracle.dequant(codes, scales, g)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert (xb.to(torch.float64).numpy() == x).all()
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    qc, qs, qg = oracle.quantize_nvfp4(bits)
    assert (qg == g).all()
    assert (qs == scales).all()
    assert (qc == codes).all()


def test_quantize_special_cases():
    K = 32
    one = 0x3F80
    # all zeros (either sign): g = 1, scales 0, codes carry the sign only
    x = np.zeros((1, 2, K), np.uint16)
    x[0, 1, 3] = 0x8000
    c, s, g = oracle.quantize_nvfp4(x)
    assert g[0] == 1.0 and (s == 0).all()
    assert c[0, 1, 1] == 0x80 and (np.delete(c.ravel(), 17) == 0).all()
    # g from the tensor amax; a block whose t rounds down saturates at 6
    x = np.zeros((1, 1, K), np.uint16)
    x[0, 0, 0] = 0x4528           # 2688: g = 1
    xv = 6.0 * 1.0625 * 1.0      # block 1: t = 1.0625 (a tie) -> s = 1.0
    x[0, 0, 16] = torch.tensor(xv, dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF
    x[0, 0, 17] = one             # 1.0 / 1.0 -> code 2
    c, s, g = oracle.quantize_nvfp4(x)
    assert g[0] == 1.0 and s[0, 0, 0] == 0x7E and s[0, 0, 1] == 0x38
    assert c[0, 0, 8] == (7 | (2 << 4))   # 6.375 -> 6 (saturated), 1.0 -> 1.0
    # each value lands on the nearest point of its block's grid +-{0..6} s_b g
    # (up to the FP32 rounding of x / s_b g at a midpoint); blocks whose scale
    # rounded down saturate at 6 s_b g
    xs = synth.normal_bf16(synth.key(6), (2, 8, 256), 0.0, 3.0)
    xs[0, 2, 40] = 0x4400          # an outlier (512)
    c, s, g = oracle.quantize_nvfp4(xs)
    deq = oracle.dequant(c, s, g)
    xd = bf16_to_f64(xs)
    sg = np.repeat(torch_e4m3(s), 16, axis=-1) * g[:, None, None]
    grid = np.array([E2M1_TABLE[c] for c in range(8)])
    nearest = np.min(np.abs(np.abs(xd)[..., None] - grid * sg[..., None]), axis=-1)
    err = np.abs(deq - xd)
    sat = np.abs(xd) > 6 * sg
    assert (err[~sat] <= nearest[~sat] + 1e-6 * np.abs(xd[~sat])).all()
    assert (np.abs(deq[sat]) == 6 * sg[sat]).all()
    assert (np.sign(deq) * np.sign(xd) >= 0).all()


# ---- router projection ----------------------------------------------------------------

@pytest.mark.parametrize("M,H,E", [(1, 16, 3), (3, 64, 9), (2, 96, 5)])
def test_router_logits_equal_exact_rational_sum(M, H, E):
    """BF16 x BF16 products of values in [2^-8, 2^8) and their sums are dyadic
    rationals float64 holds exactly: the oracle must equal the exact sum."""
    rng = np.random.default_rng(900 + M * 10 + H + E)
    x = _bf16_bits_in_range(rng, (M, H))
    wr = _bf16_bits_in_range(rng, (E, H))
    xf = [[Fraction(float(v)) for v in row] for row in bf16_to_f64(x)]
    wf = [[Fraction(float(v)) for v in row] for row in bf16_to_f64(wr)]
    got = oracle.router_logits(x, wr)
    for m in range(M):
        for e in range(E):
            exact = sum(xf[m][h] * wf[e][h] for h in range(H))
            assert got[m, e] == float(exact) and Fraction(got[m, e]) == exact, (m, e)


def test_router_logits_special_cases():
    M, H, E = 3, 128, 6
    x = synth.normal_bf16(synth.key(4), (M, H))
    xd = bf16_to_f64(x)
    # row e of W_r one-hot at column c_e (value 2^-e): logits pick x's columns
    wr = np.zeros((E, H), np.uint16)
    cols = [0, 5, 64, 100, 127, 31]
    for e, c in enumerate(cols):
        wr[e, c] = (127 - e) << 7  # 2^-e
    got = oracle.router_logits(x, wr)
    for e, c in enumerate(cols):
        assert (got[:, e] == xd[:, c] * 2.0 ** -e).all()
    # swapping rows of W_r swaps the logit columns; negating x negates them
    wr = synth.normal_bf16(synth.key(5), (E, H))
    a = oracle.router_logits(x, wr)
    b = oracle.router_logits(x, wr[::-1].copy())
    assert (b == a[:, ::-1]).all()
    assert (oracle.router_logits(x ^ np.uint16(0x8000), wr) == -a).all()


# ---- FP8 skinny product (Elsa page, "An FP8 fast path") ------------------------------

@pytest.mark.parametrize("M,K,N,sexp", [(1, 16, 1, 0), (2, 48, 5, -9), (3, 64, 7, 4)])
def test_gemm_fp8_equals_exact_rational_sum(M, K, N, sexp):
    """Every finite E4M3 code (incl. subnormals and negatives) times BF16 values
    in [2^-8, 2^8): each product and partial sum is a dyadic rational float64
    holds, so the oracle must equal the exact sum, decoded with torch's own
    float8_e4m3fn, bit for bit."""
    rng = np.random.default_rng(7000 + M * 100 + K + N)
    x = _bf16_bits_in_range(rng, (M, K))
    w = rng.choice(FINITE_E4M3, (N, K)).astype(np.uint8)
    s = 2.0 ** sexp
    xf = [[Fraction(float(v)) for v in row] for row in bf16_to_f64(x)]
    wv = torch_e4m3(w)
    got = oracle.gemm_fp8(x, w, s)
    for m in range(M):
        for n in range(N):
            exact = sum(xf[m][k] * Fraction(float(wv[n, k])) for k in range(K)) * Fraction(s)
            assert got[m, n] == float(exact) and Fraction(got[m, n]) == exact, (m, n)


def test_gemm_fp8_special_cases():
    M, K, N = 3, 64, 5
    x = synth.normal_bf16(synth.key(2), (M, K))
    xd = bf16_to_f64(x)
    # one non-zero weight in row 2, column 41: 0xC3 = -(1 + 3/8) * 2^1
    w = np.zeros((N, K), np.uint8)
    w[2, 41] = 0xC3
    y = oracle.gemm_fp8(x, w, 0.125)
    assert (y[:, [0, 1, 3, 4]] == 0).all()
    assert (y[:, 2] == xd[:, 41] * -2.75 * 0.125).all()
    # unit rows of x read back the decoded weights exactly (every finite code)
    K2 = 256
    eye = np.zeros((4, K2), np.uint16)
    cols = [0, 17, 130, 255]
    for r, c in enumerate(cols):
        eye[r, c] = 0x3F80  # 1.0
    w = np.zeros((254, K2), np.uint8)
    for r, c in enumerate(cols):
        w[:, c] = FINITE_E4M3
    y = oracle.gemm_fp8(eye, w, 1.0)
    ref = torch_e4m3(FINITE_E4M3.astype(np.uint8))
    for r in range(4):
        assert (y[r] == ref).all()
    # 0x80 is -0 and adds nothing; scaling s scales y exactly
    rng = np.random.default_rng(5)
    w = rng.choice(FINITE_E4M3, (N, K)).astype(np.uint8)
    wz = w.copy()
    wz[:, ::3] = 0x80
    wz0 = w.copy()
    wz0[:, ::3] = 0
    assert (oracle.gemm_fp8(x, wz, 1.0) == oracle.gemm_fp8(x, wz0, 1.0)).all()
    assert (oracle.gemm_fp8(x, w, 0.75) * 2 == oracle.gemm_fp8(x, w, 1.5)).all()


# ---- routing -------------------------------------------------------------------------

def _brute_route(logits, k, bias=None):
    M, E = logits.shape
    ids, ws = [], []
    for m in range(M):
        lp = logits[m] if bias is None else (logits[m] + bias).astype(np.float32)
        key = lambda e: (1 if math.isnan(lp[e]) else 0, 0.0 if math.isnan(lp[e]) else -float(lp[e]), e)
        order = sorted(range(E), key=key)[:k]
        ids.append(order)
    return np.array(ids, dtype=np.int32)


@pytest.mark.parametrize("M,E,k,seed,bias", [(1, 256, 8, 0, False), (4, 256, 8, 1, False),
                                             (16, 256, 8, 2, True), (5, 64, 2, 3, False),
                                             (3, 256, 1, 4, True), (7, 8, 8, 5, False)])
def test_route_matches_brute_force_sort(M, E, k, seed, bias):
    logits = synth.normal_f32(synth.key(seed, 9), (M, E))
    b = synth.normal_f32(synth.key(seed, 10), (E,), 0.0, 0.5) if bias else None
    ids, w = oracle.route_topk(logits, k, b)
    assert (ids == _brute_route(logits, k, b)).all()
    for m in range(M):
        assert len(set(ids[m])) == k
        assert abs(math.fsum(w[m]) - 1.0) <= 1e-12
        assert all(w[m][j] >= w[m][j + 1] for j in range(k - 1))
        lp = logits[m] if b is None else (logits[m] + b).astype(np.float32)
        for j in range(1, k):   # closed-form ratio of softmax weights
            r = math.exp(float(lp[ids[m][j]]) - float(lp[ids[m][0]]))
            assert abs(w[m][j] / w[m][0] - r) <= 1e-12 * max(1.0, r)


def test_route_ties_zeros_and_nan():
    E, k = 16, 4
    rows = np.array([
        [1.0] * E,                                            # all equal -> 0..3
        [0.0, -0.0, 0.0, -0.0] + [-1.0] * 12,                 # +/-0 tie -> index order
        [np.nan, 2.0, np.nan, 2.0, 1.0, -np.inf] + [-3.0] * 10,
        [-np.inf] * 2 + [5.0, 5.0, 5.0] + [-np.inf] * 11,
    ], dtype=np.float32)
    ids, w = oracle.route_topk(rows, k)
    assert ids[0].tolist() == [0, 1, 2, 3]
    assert ids[1].tolist() == [0, 1, 2, 3]
    assert ids[2].tolist() == [1, 3, 4, 6]
    assert ids[3].tolist() == [2, 3, 4, 0]
    assert np.allclose(w[0], 0.25, rtol=0, atol=1e-15)
    assert np.allclose(w[3], [1 / 3, 1 / 3, 1 / 3, 0.0], rtol=0, atol=1e-15)
    assert (ids == _brute_route(rows, k)).all()
    # fp32 bias add decides ties that exact arithmetic would not
    # exactly, 1 + 0.75 ulp < 1 + 1 ulp puts expert 1 first; in FP32 the sum
    # rounds up to 1 + 1 ulp, the two tie, and the lower index wins
    lg = np.array([[1.0, 1.0 + 2 ** -23, 0.0, 0.0]], np.float32)
    b = np.array([3 * 2 ** -25, 0.0, 0.0, 0.0], np.float32)
    ids, _ = oracle.route_topk(lg, 1, b)
    assert ids[0, 0] == 0
    with pytest.raises(ValueError):
        oracle.route_topk(rows, 17)


def test_group_by_expert_matches_brute_counting_sort():
    for seed, (M, E, k) in enumerate([(4, 256, 8), (16, 256, 8), (256, 256, 8), (3, 5, 2)]):
        logits = synth.normal_f32(synth.key(seed, 12), (M, E))
        ids, _ = oracle.route_topk(logits, k)
        counts, offsets, pairs, active, active_offsets, na = oracle.group_by_expert(ids, E)
        flat = ids.reshape(-1)
        assert (counts == np.bincount(flat, minlength=E)).all()
        assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
        assert counts.sum() == M * k and offsets[-1] == M * k
        assert sorted(pairs.tolist()) == list(range(M * k))
        brute = [p for e in range(E) for p in range(M * k) if flat[p] == e]
        assert pairs.tolist() == brute
        for e in range(E):
            grp = pairs[offsets[e]:offsets[e + 1]]
            assert (flat[grp] == e).all() and (np.diff(grp) > 0).all()
        assert na == int((counts > 0).sum())
        assert active[:na].tolist() == [e for e in range(E) if counts[e] > 0]
        assert (active[na:] == -1).all()
        # per-slot run starts: slot s's pairs are pairs[active_offsets[s]:active_offsets[s+1]]
        for s_ in range(na):
            run = pairs[active_offsets[s_]:active_offsets[s_ + 1]]
            assert len(run) == counts[active[s_]] and (flat[run] == active[s_]).all()
        assert (active_offsets[na:] == M * k).all()


# ---- expert FFN and MoE block ----------------------------------------------------------

def _onehot_layer(H, I, E, x, a, b, c, vcode, scode, g_gu, g_dn):
    """Expert e's gate row i reads x[a[e][i]], up row i reads x[b[e][i]], down
    row n reads h[c[e][n]]; the single non-zero weight is e2m1(vcode) *
    e4m3(scode) * g."""
    gu_c = np.zeros((E, 2 * I, H // 2), np.uint8)
    gu_s = np.full((E, 2 * I, H // 16), 0x38, np.uint8)
    dn_c = np.zeros((E, H, I // 2), np.uint8)
    dn_s = np.full((E, H, I // 16), 0x38, np.uint8)

    def put(cd, sc, e, row, col):
        cd[e, row, col // 2] |= (vcode << 4) if col & 1 else vcode
        sc[e, row, col // 16] = scode

    for e in range(E):
        for i in range(I):
            put(gu_c, gu_s, e, i, a[e][i])
            put(gu_c, gu_s, e, I + i, b[e][i])
        for n in range(H):
            put(dn_c, dn_s, e, n, c[e][n])
    gu = NVFP4(gu_c, gu_s, np.full(E, g_gu, np.float32))
    dn = NVFP4(dn_c, dn_s, np.full(E, g_dn, np.float32))
    return gu, dn


def test_moe_block_closed_form_onehot():
    """Closed form of a constructed block: y_e[n] = wv*g_dn * silu(wv*g_gu*x[a]) *
    (wv*g_gu*x[b]) with a = a_e[c_e[n]], b = b_e[c_e[n]]; out = sum_j w_j y + residual.
    Pins the gate/up split, nibble and scale-block positions, the combine and
    the residual."""
    H, I, E, M, k = 64, 16, 3, 2, 2
    rng = np.random.default_rng(3)
    x = synth.normal_bf16(synth.key(3, 1), (M, H))
    res = synth.normal_bf16(synth.key(3, 2), (M, H))
    a = [rng.integers(0, H, I) for _ in range(E)]
    b = [rng.integers(0, H, I) for _ in range(E)]
    c = [rng.integers(0, I, H) for _ in range(E)]
    vcode, scode = 13, 0x31  # -3.0, 0.5625
    wv = -3.0 * 0.5625
    gu, dn = _onehot_layer(H, I, E, x, a, b, c, vcode, scode, 0.5, 0.25)
    ids = np.array([[2, 0], [1, 2]], np.int32)
    w = np.array([[0.7, 0.3], [0.25, 0.75]])
    out = oracle.moe_block(x, ids, w, gu, dn, residual=res)
    xd, rd = bf16_to_f64(x), bf16_to_f64(res)
    silu = lambda t: t / (1.0 + math.exp(-t))
    for m in range(M):
        for n in range(H):
            terms = []
            for j in range(k):
                e = ids[m, j]
                i = c[e][n]
                ug = wv * 0.5 * xd[m, a[e][i]]
                uu = wv * 0.5 * xd[m, b[e][i]]
                terms.append(w[m, j] * wv * 0.25 * silu(ug) * uu)
            ref = terms[0] + terms[1] + rd[m, n]
            assert abs(out[m, n] - ref) <= 1e-14 * max(1.0, abs(ref)), (m, n)


def _decimal_block(layer: MoELayer, ids, w, prec=40):
    """Brute force of the block in 40-digit decimal arithmetic on the dequantized
    weights from the independent decoders."""
    getcontext().prec = prec
    M, H, I = layer.M, layer.H, layer.I
    xd = bf16_to_f64(layer.x)

    def deq(t: NVFP4, e):
        v = table_e2m1(unpack_nibbles(t.codes[e]))
        s = np.repeat(torch_e4m3(t.scales[e]), 16, axis=-1)
        return v * s * float(t.g[e])  # exact in double (dyadic, few bits)

    def ffn(xrow, Wgu, Wdn):
        u = [sum(Decimal(float(xrow[kk])) * Decimal(float(Wgu[n, kk])) for kk in range(H))
             for n in range(2 * I)]
        h = [u[i] / (1 + (-u[i]).exp()) * u[I + i] for i in range(I)]
        return [sum(h[i] * Decimal(float(Wdn[n, i])) for i in range(I)) for n in range(H)]

    out = [[Decimal(0)] * H for _ in range(M)]
    for m in range(M):
        for j in range(ids.shape[1]):
            e = int(ids[m, j])
            y = ffn(xd[m], deq(layer.gate_up, e), deq(layer.down, e))
            for n in range(H):
                out[m][n] += Decimal(float(w[m, j])) * y[n]
        if layer.shared_gate_up is not None:
            y = ffn(xd[m], deq(layer.shared_gate_up, 0), deq(layer.shared_down, 0))
            for n in range(H):
                out[m][n] += y[n]
    return np.array([[float(v) for v in row] for row in out])


def test_moe_block_decimal_brute_force():
    lay = moe_layer(seed=7, wl=90, M=2, E_=6, H_=32, I_=16, k=2, shared=True)
    ids, w = oracle.route_topk(lay.logits, lay.k)
    out = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down)
    ref = _decimal_block(lay, ids, w)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    # and through the whole step from logits
    ids2, w2, out2 = oracle.moe_decode(lay.x, lay.logits, lay.k, lay.gate_up, lay.down,
                                       shared_gate_up=lay.shared_gate_up,
                                       shared_down=lay.shared_down)
    assert (ids2 == ids).all() and (w2 == w).all() and (out2 == out).all()


def test_moe_block_invariants():
    lay = moe_layer(seed=8, wl=91, M=3, E_=8, H_=64, I_=32, k=2)
    ids, w = oracle.route_topk(lay.logits, lay.k)
    base = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down)
    # rows are independent
    for m in range(lay.M):
        one = oracle.moe_block(lay.x[m:m + 1], ids[m:m + 1], w[m:m + 1], lay.gate_up, lay.down)
        assert (one[0] == base[m]).all()
    # down is linear: doubling its tensor scale doubles the output exactly,
    # flipping every down sign bit negates it exactly
    dn2 = NVFP4(lay.down.codes, lay.down.scales, lay.down.g * 2)
    assert (oracle.moe_block(lay.x, ids, w, lay.gate_up, dn2) == 2 * base).all()
    dneg = NVFP4(lay.down.codes ^ np.uint8(0x88), lay.down.scales, lay.down.g)
    assert (oracle.moe_block(lay.x, ids, w, lay.gate_up, dneg) == -base).all()
    # k = 1, weight 1 is one expert FFN
    e = int(ids[0, 0])
    one = oracle.moe_block(lay.x[:1], np.array([[e]], np.int32), np.ones((1, 1)), lay.gate_up,
                           lay.down)
    y = oracle.expert_ffn(lay.x[0], lay.gate_up.select([e]), lay.down.select([e]))
    assert (one[0] == y).all()
    # gate rows at zero switch the expert off: silu(0) * up = 0
    gz = lay.gate_up.codes.copy()
    gz[:, :lay.I, :] = 0
    gu0 = NVFP4(gz, lay.gate_up.scales, lay.gate_up.g)
    assert (oracle.moe_block(lay.x, ids, w, gu0, lay.down) == 0).all()
    # a zero shared expert adds exactly nothing
    zgu = NVFP4(np.zeros((1, 2 * lay.I, lay.H // 2), np.uint8),
                np.full((1, 2 * lay.I, lay.H // 16), 0x38, np.uint8), np.ones(1, np.float32))
    zdn = NVFP4(np.zeros((1, lay.H, lay.I // 2), np.uint8),
                np.full((1, lay.H, lay.I // 16), 0x38, np.uint8), np.ones(1, np.float32))
    assert (oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, zgu, zdn) == base).all()


def test_moe_block_touched_subset_equals_full():
    lay = moe_layer(seed=9, wl=92, M=4, E_=32, H_=64, I_=32, k=4)
    ids, w = oracle.route_topk(lay.logits, lay.k)
    full = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down)
    sub = oracle.moe_block_touched(lay, ids, w)
    assert (full == sub).all()
    rows = oracle.moe_block_touched(lay, ids, w, rows=[1, 3])
    assert (rows == full[[1, 3]]).all()


@pytest.mark.parametrize("threads", [2, 3, 8])
def test_threaded_oracle_is_bit_identical(threads):
    """The thread split changes nothing: every output of the products and of
    the MoE block (experts with more pairs than one job takes, a shared
    expert over more rows than one job takes, a residual) equals the
    single-threaded result bit for bit."""
    lay = moe_layer(seed=10, wl=93, M=37, E_=12, H_=256, I_=64, k=3, shared=True)
    ids, w = oracle.route_topk(lay.logits, lay.k)
    res = synth.normal_bf16(synth.key(10, 94), (lay.M, lay.H))
    rng = np.random.default_rng(3)
    x = synth.normal_bf16(synth.key(10, 95), (5, 256))
    wc = rng.integers(0, 256, (1, 300, 128), dtype=np.uint8)
    ws = rng.integers(0x18, 0x58, (1, 300, 16), dtype=np.uint8)
    w8 = rng.integers(0, 0x7F, (300, 256), dtype=np.uint8)
    wr = synth.normal_bf16(synth.key(10, 96), (40, 256))

    def run():
        return [oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                                 lay.shared_down, res),
                oracle.gemm(x, wc[0], ws[0], 0.37), oracle.gemm_fp8(x, w8, 0.5),
                oracle.router_logits(x, wr)]

    saved = oracle.threads()
    try:
        oracle.set_threads(1)
        one = run()
        oracle.set_threads(threads)
        assert oracle.threads() == threads
        many = run()
    finally:
        oracle.set_threads(saved)
    for a, b in zip(one, many):
        assert a.view(np.uint64).tobytes() == b.view(np.uint64).tobytes()


def test_moe_block_f64_on_bf16_values_equals_moe_block():
    """The float64-input block is the same computation: on BF16-valued rows and
    residual it gives moe_block's result bit for bit, and its rows stay
    independent for values off the BF16 grid."""
    lay = moe_layer(seed=11, wl=97, M=3, E_=8, H_=64, I_=32, k=2, shared=True)
    ids, w = oracle.route_topk(lay.logits, lay.k)
    res = synth.normal_bf16(synth.key(11, 98), (lay.M, lay.H))
    a = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                         lay.shared_down, res)
    b = oracle.moe_block_f64(bf16_to_f64(lay.x), ids, w, lay.gate_up, lay.down,
                             lay.shared_gate_up, lay.shared_down, bf16_to_f64(res))
    assert (a == b).all()
    xf = bf16_to_f64(lay.x) * (1 + 2.0 ** -20)  # not representable in BF16
    full = oracle.moe_block_f64(xf, ids, w, lay.gate_up, lay.down)
    for m in range(lay.M):
        one = oracle.moe_block_f64(xf[m:m + 1], ids[m:m + 1], w[m:m + 1], lay.gate_up,
                                   lay.down)
        assert (one[0] == full[m]).all()
