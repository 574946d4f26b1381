"""GPU parity of each kernel against the oracle, through the C ABI.

Decode and routing are compared bit for bit; products under
|gpu - ref| <= 1e-2 |ref| + 1e-3 against the oracle's float64 result.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import NVFP4, dense_skinny, moe_layer
from tests.helpers import (check_routing_exact, dev_bf16_to_f64, pack, to_dev_bf16,
                           tol_ratio, upload_layer)

pytestmark = pytest.mark.gpu

FINITE_E4M3 = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)


@pytest.fixture(scope="module")
def m(gpu):
    import nvfp4_moe_skinny_amd as m
    return m


def _all_codes_all_scales(G, N, K, gvals, seed=0):
    """Every 16-element block enumerates the 16 E2M1 codes; the scales cycle
    through every finite E4M3 code (with a per-row offset)."""
    codes = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8),
                    (G, N, K // 16))
    nb = K // 16
    idx = (np.arange(G * N * nb).reshape(G, N, nb) + seed) % len(FINITE_E4M3)
    scales = FINITE_E4M3[idx]
    return NVFP4(codes, scales, np.asarray(gvals, np.float32))


@pytest.mark.parametrize("K,N", [(2048, 8), (2048, 11), (512, 33), (64, 300), (32, 513),
                                 (1024, 16), (128, 128),
                                 # several panels: K = 3 x 32, 5 x 32, 3 x 512, 3 x 1024, 2 x 2048
                                 (96, 700), (160, 513), (1536, 40), (3072, 17), (4096, 9)])
@pytest.mark.parametrize("path", [0, 1])
def test_dequant_bit_exact_every_code_and_scale(m, gpu, K, N, path):
    nv = _all_codes_all_scales(3, N, K, [1.0, 2.0 ** -9, 0.37], seed=K + N)
    pw = pack(nv, gpu, m)
    for apply_g in (True, False):
        got = m.nvfp4_dequant_f32(pw, apply_g=apply_g, path=path).cpu().numpy()
        g = nv.g if apply_g else np.ones_like(nv.g)
        ref = oracle.dequant_f32(nv.codes, nv.scales, g)
        assert (got.view(np.uint32) == ref.view(np.uint32)).all()


def test_dequant_random_tensor(m, gpu):
    rng = np.random.default_rng(1)
    G, N, K = 4, 77, 256
    nv = NVFP4(rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8),
               rng.choice(FINITE_E4M3, (G, N, K // 16)).astype(np.uint8),
               np.array([1.0, 0.5, 3.0, 2.0 ** -8], np.float32))
    pw = pack(nv, gpu, m)
    got = m.nvfp4_dequant_f32(pw, path=0).cpu().numpy()
    ref = oracle.dequant_f32(nv.codes, nv.scales, nv.g)
    assert (got.view(np.uint32) == ref.view(np.uint32)).all()


@pytest.mark.parametrize("M,K,N,g", [(1, 2048, 512, 1.0),      # the single dense matrix
                                     (8, 2048, 64, 2.0 ** -9),  # per-layer 2048 -> 64
                                     (3, 2048, 37, 0.37), (19, 512, 100, 1.0),
                                     (5, 256, 64, 2.0 ** -4), (2, 32, 700, 1.0),
                                     (16, 1024, 48, 0.5), (4, 64, 5, 1.0),
                                     # MFMA path (K = 2048, M >= 4): odd tile counts,
                                     # ragged N, one and several 16-row passes over x
                                     (4, 2048, 8, 2.0 ** -9), (5, 2048, 24, 1.0),
                                     (16, 2048, 100, 0.37), (17, 2048, 40, 1.0),
                                     (33, 2048, 17, 2.0 ** -9), (6, 2048, 4104, 1.0),
                                     # K split over four waves: N <= 4096, M <= 16
                                     (12, 2048, 4096, 1.0), (7, 2048, 1, 0.5),
                                     # K % 32 == 0 beyond powers of two (several panels)
                                     (1, 96, 600, 1.0), (3, 96, 1025, 0.5), (9, 160, 70, 1.0),
                                     (1, 1536, 512, 2.0 ** -8), (5, 3072, 300, 2.0 ** -9),
                                     (6, 4096, 2048, 2.0 ** -9), (17, 4096, 33, 1.0),
                                     (2, 2016, 40, 1.0), (8, 6144, 100, 2.0 ** -9)])
def test_skinny_gemm(m, gpu, M, K, N, g):
    x, w = dense_skinny(seed=0, M=M, K=K, N=N, g=g)
    pw = pack(w, gpu, m)
    y = m.nvfp4_skinny_gemm(to_dev_bf16(x, gpu), pw)
    torch.cuda.synchronize()
    ref = oracle.gemm(x, w.codes[0], w.scales[0], g)
    assert tol_ratio(dev_bf16_to_f64(y), ref) <= 1.0


@pytest.mark.parametrize("M,E,k,bias", [(1, 256, 8, False), (4, 256, 8, False),
                                        (8, 256, 8, False), (16, 256, 8, True),
                                        (64, 256, 8, True), (65, 256, 8, False),
                                        (256, 256, 8, False), (1024, 256, 8, False),
                                        (3, 5, 2, False), (7, 64, 1, True), (20, 8, 8, False),
                                        (64, 8, 8, False),  # every row takes every expert
                                        (2048, 64, 4, True), (8192, 256, 1, False),  # > 1024 rows
                                        (33, 3, 3, True),
                                        (5, 1, 1, True)])  # one expert: every row, w = 1
def test_route_bit_exact(m, gpu, M, E, k, bias):
    for seed in range(3):
        lg = synth.normal_f32(synth.key(seed, 100, M, E), (M, E))
        b = synth.normal_f32(synth.key(seed, 101, E), (E,), 0.0, 0.5) if bias else None
        r = m.moe_route_topk(torch.from_numpy(lg).to(gpu), k,
                             None if b is None else torch.from_numpy(b).to(gpu))
        torch.cuda.synchronize()
        ids, w = oracle.route_topk(lg, k, b)
        check_routing_exact(r, ids, w, E)


def test_route_zipf_logits(m, gpu):
    lg = synth.zipf_gumbel_logits(synth.key(0, 102), synth.key(0, 103), 256, 256, 1.1)
    r = m.moe_route_topk(torch.from_numpy(lg).to(gpu), 8)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(lg, 8)
    check_routing_exact(r, ids, w, 256)


def test_route_constructed_ties(m, gpu):
    E, k = 16, 4
    rows = np.array([
        [1.0] * E,
        [0.0, -0.0, 0.0, -0.0] + [-1.0] * 12,
        [np.nan, 2.0, np.nan, 2.0, 1.0, -np.inf] + [-3.0] * 10,
        [-np.inf] * 2 + [5.0, 5.0, 5.0] + [-np.inf] * 11,
        [-0.0] * E,
        [3.0, 3.0, -0.0, 0.0] + [2.0] * 12,
    ], dtype=np.float32)
    r = m.moe_route_topk(torch.from_numpy(rows).to(gpu), k)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(rows, k)
    check_routing_exact(r, ids, w, E)
    # the FP32 bias add decides a tie that exact arithmetic would not
    lg = np.array([[1.0, 1.0 + 2 ** -23, 0.0, 0.0]], np.float32)
    b = np.array([3 * 2 ** -25, 0.0, 0.0, 0.0], np.float32)
    r = m.moe_route_topk(torch.from_numpy(lg).to(gpu), 1, torch.from_numpy(b).to(gpu))
    torch.cuda.synchronize()
    assert int(r.ids.cpu()[0, 0]) == 0


def _run_block(m, gpu, lay, residual=None, **kw):
    d = upload_layer(lay, gpu, m)
    r = m.moe_route_topk(d["logits"], lay.k, d["bias"])
    res = None if residual is None else to_dev_bf16(residual, gpu)
    out = m.moe_nvfp4_decode(d["x"], r, d["gu"], d["dn"], d["sgu"], d["sdn"], residual=res, **kw)
    torch.cuda.synchronize()
    return r, dev_bf16_to_f64(out)


@pytest.mark.parametrize("schedule", [2, 3])
@pytest.mark.parametrize("M,E,H,I,k,shared,resid", [
    (1, 16, 256, 256, 4, False, False), (3, 16, 256, 256, 4, True, False),
    (8, 16, 256, 512, 4, False, True), (17, 16, 512, 256, 4, True, True),
    (5, 8, 512, 512, 8, True, False), (2, 32, 1024, 256, 2, False, True),
    (6, 4, 2048, 512, 1, True, True), (11, 256, 256, 256, 8, False, False),
    (70, 64, 2048, 512, 8, True, True), (33, 40, 1024, 1024, 3, False, False),
    (4, 256, 2048, 2048, 8, False, False), (16, 8, 2048, 256, 8, True, False),
    (3, 1, 256, 256, 1, True, False),  # a single expert (k = E = 1)
    (40, 1, 2048, 512, 1, True, False)])  # one routed slot of 40 rows beside the shared one
def test_moe_block_small(m, gpu, M, E, H, I, k, shared, resid, schedule):
    lay = moe_layer(seed=M + E, wl=200, M=M, E_=E, H_=H, I_=I, k=k, shared=shared)
    residual = synth.normal_bf16(synth.key(5, 201, M), (M, H)) if resid else None
    # the two-launch schedule takes any M once no slot uses MFMA
    kw = dict(dense_min_rows=M + 1) if schedule == 3 else {}
    r, out = _run_block(m, gpu, lay, residual, schedule=schedule, **kw)
    ids, w = oracle.route_topk(lay.logits, k, lay.bias)
    check_routing_exact(r, ids, w, E)
    ref = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, residual)
    assert tol_ratio(out, ref) <= 1.0


@pytest.mark.parametrize("M,E,H,I,k,shared,resid,bias", [
    (1, 256, 2048, 512, 8, False, False, False), (4, 256, 2048, 512, 8, False, False, True),
    (8, 256, 2048, 512, 8, True, True, True), (3, 16, 256, 256, 4, True, False, False),
    (5, 8, 512, 512, 8, True, False, False), (2, 32, 1024, 256, 2, False, True, False),
    (12, 64, 2048, 512, 8, True, False, True), (6, 4, 2048, 512, 1, True, True, False),
    # three routed slots without a shared expert at H = 2048, I = 512: three-wave
    # down blocks, each wave restaging its own x and h rows through LDS
    (5, 64, 2048, 512, 3, False, True, True),
    # down tiles of more than 64 output rows (I = 128: 128, I = 96: 512)
    (4, 16, 512, 128, 4, False, True, True), (3, 8, 2048, 96, 2, True, True, False),
    # beyond M = 15 with dense_min_rows above M
    (16, 64, 2048, 512, 8, False, False, False), (24, 32, 2048, 512, 4, True, True, True)])
def test_moe_route_decode_fused(m, gpu, M, E, H, I, k, shared, resid, bias):
    """Routing inside the gate_up launch: ids and w bit-identical to the oracle's
    routing, the output within tolerance of the oracle and bit-identical to
    moe_route_topk + moe_nvfp4_decode with the two-launch schedule."""
    lay = moe_layer(seed=M + 3 * E, wl=205, M=M, E_=E, H_=H, I_=I, k=k, bias=bias, shared=shared)
    residual = synth.normal_bf16(synth.key(5, 206, M), (M, H)) if resid else None
    d = upload_layer(lay, gpu, m)
    res = None if residual is None else to_dev_bf16(residual, gpu)
    dmr = M + 1 if M >= 12 else 0
    ws = m.moe_workspace(M, E, k, H, I, shared, gpu)
    call = lambda: m.moe_nvfp4_route_decode(d["x"], d["logits"], k, d["gu"], d["dn"], d["bias"],
                                            d["sgu"], d["sdn"], residual=res, workspace=ws,
                                            dense_min_rows=dmr)
    out, ids_d, w_d = call()
    again, _, _ = call()  # the same workspace again
    r = m.moe_route_topk(d["logits"], k, d["bias"])
    out2 = m.moe_nvfp4_decode(d["x"], r, d["gu"], d["dn"], d["sgu"], d["sdn"], residual=res,
                              schedule=3, dense_min_rows=dmr)
    torch.cuda.synchronize()
    ids, w = oracle.route_topk(lay.logits, k, lay.bias)
    assert (ids_d.cpu().numpy() == ids).all()
    assert np.max(np.abs(w_d.cpu().numpy().astype(np.float64) - w)) <= 1e-6
    assert torch.equal(w_d.view(torch.int32), r.w.view(torch.int32))
    ref = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, residual)
    assert tol_ratio(dev_bf16_to_f64(out), ref) <= 1.0
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(again.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("M,k,shared,N", [(4, 8, False, 64), (8, 8, True, 64), (1, 4, False, 8),
                                         (6, 3, True, 100), (12, 8, True, 4096)])
def test_moe_route_decode_with_projection(m, gpu, M, k, shared, N):
    """A dense projection of x computed by blocks of the down launch: bit-identical
    to nvfp4_skinny_gemm of the same x, and the block's own outputs unchanged."""
    lay = moe_layer(seed=M + N, wl=207, M=M, E_=64, H_=2048, I_=512, k=k, shared=shared)
    _, pw_h = dense_skinny(seed=M, M=M, K=2048, N=N, g=2.0 ** -9)
    d = upload_layer(lay, gpu, m)
    pw = pack(pw_h, gpu, m)
    args = (d["x"], d["logits"], k, d["gu"], d["dn"], None, d["sgu"], d["sdn"])
    out0, ids0, w0 = m.moe_nvfp4_route_decode(*args)
    py = torch.full((M, N), 7, dtype=torch.int16, device=gpu).view(torch.bfloat16)
    out1, ids1, w1 = m.moe_nvfp4_route_decode(*args, proj=pw, proj_out=py)
    ref = m.nvfp4_skinny_gemm(d["x"], pw)
    torch.cuda.synchronize()
    assert torch.equal(py.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(ids0, ids1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    pref = oracle.gemm(lay.x, pw_h.codes[0], pw_h.scales[0], float(pw_h.g[0]))
    assert tol_ratio(dev_bf16_to_f64(py), pref) <= 1.0


@pytest.mark.parametrize("M,E,H,I,k,shared,resid", [
    (4, 16, 1536, 768, 8, True, True),     # gate 3 panels of 512, down 3 panels of 256
    (3, 8, 96, 512, 2, True, False),       # gate one chunk per row and panel (L = 1), 3 panels
    (5, 8, 160, 512, 4, False, True),      # 5 panels of 32; down rows past H in the last block
    (6, 16, 2560, 1408, 8, True, False),   # down 11 panels of 128 (L = 4: two rows a lane)
    (2, 4, 4096, 1024, 2, False, True),    # gate 2 panels of 2048
    (20, 8, 1536, 768, 4, True, True),     # more rows: the expert-major launches
    (40, 4, 96, 512, 2, True, False),
    (3, 8, 128, 256, 2, False, True)])     # one panel of 128: four lanes a row (L = 4)
@pytest.mark.parametrize("entry", ["decode", "decode3", "route_decode"])
def test_moe_block_panel_shapes(m, gpu, M, E, H, I, k, shared, resid, entry):
    """H and I that are multiples of 32 but not powers of two up to 2048 (the
    matrices split into several panels, some with fewer than eight lanes per
    row): every schedule against the oracle, every element."""
    lay = moe_layer(seed=M + H + I, wl=208, M=M, E_=E, H_=H, I_=I, k=k, shared=shared,
                    bias=shared)
    residual = synth.normal_bf16(synth.key(5, 209, M), (M, H)) if resid else None
    d = upload_layer(lay, gpu, m)
    res = None if residual is None else to_dev_bf16(residual, gpu)
    if entry == "route_decode":
        out, ids_d, w_d = m.moe_nvfp4_route_decode(d["x"], d["logits"], k, d["gu"], d["dn"],
                                                   d["bias"], d["sgu"], d["sdn"], residual=res)
        torch.cuda.synchronize()
        ids, w = oracle.route_topk(lay.logits, k, lay.bias)
        assert (ids_d.cpu().numpy() == ids).all()
    else:
        r, got = _run_block(m, gpu, lay, residual, schedule=3 if entry == "decode3" else 0)
        ids, w = oracle.route_topk(lay.logits, k, lay.bias)
        check_routing_exact(r, ids, w, E)
    if entry == "route_decode":
        got = dev_bf16_to_f64(out)
    ref = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, residual)
    assert tol_ratio(got, ref) <= 1.0


@pytest.mark.parametrize("M,E,k,shared,resid,dense_min_rows", [
    (6, 4, 1, True, True, 1),      # every slot on MFMA, most blocks with one row
    (17, 8, 8, True, False, 16),   # each expert holds all 17 rows: a 1-row second block
    (48, 2, 2, True, False, 16),   # 48 rows: two passes over column blocks
    (40, 3, 2, False, True, 8),    # MFMA and VALU slots side by side
    (33, 64, 8, True, True, 4),
    # more rows: the wide kernels (2 or 4 rows per VALU batch, MFMA passes in turn)
    (64, 4, 2, True, True, 16),    # every slot on MFMA, ragged last passes
    (100, 16, 4, True, False, 8),  # MFMA and VALU slots, a 7-pass shared expert
    (72, 256, 8, False, True, 4)])  # up to 256 active slots
def test_moe_block_dense_mfma(m, gpu, M, E, k, shared, resid, dense_min_rows):
    """Three-launch schedule at H = 2048, I = 512, where slots with at least
    dense_min_rows rows run on BF16 MFMA (exact BF16 weights, h as hi + lo)."""
    lay = moe_layer(seed=7 * M + E, wl=203, M=M, E_=E, H_=2048, I_=512, k=k, shared=shared)
    residual = synth.normal_bf16(synth.key(5, 204, M), (M, 2048)) if resid else None
    r, out = _run_block(m, gpu, lay, residual, schedule=2, dense_min_rows=dense_min_rows)
    ids, w = oracle.route_topk(lay.logits, k, lay.bias)
    check_routing_exact(r, ids, w, E)
    ref = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, residual)
    assert tol_ratio(out, ref) <= 1.0


@pytest.mark.parametrize("M,E,k,shared", [(16, 8, 8, True), (13, 4, 2, False), (7, 3, 3, True),
                                          (15, 16, 5, True)])
def test_moe_block_valu_rows_small_m(m, gpu, M, E, k, shared):
    """M <= 16, three launches with every slot on VALU (threshold above M):
    slots of up to 16 rows through the one-row gate_up items and the down
    kernel's two-row batches, odd counts included, every element."""
    lay = moe_layer(seed=11 * M + E, wl=205, M=M, E_=E, H_=2048, I_=512, k=k, shared=shared)
    residual = synth.normal_bf16(synth.key(5, 206, M), (M, 2048))
    r, out = _run_block(m, gpu, lay, residual, schedule=2, dense_min_rows=M + 1)
    ids, w = oracle.route_topk(lay.logits, k, lay.bias)
    check_routing_exact(r, ids, w, E)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() >= 3
    ref = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, residual)
    assert tol_ratio(out, ref) <= 1.0


@pytest.mark.parametrize("M", [9, 12, 24, 33, 48])
def test_moe_block_default_threshold_zipf(m, gpu, M):
    """The library's default MFMA threshold, which depends on M (3 rows for
    9 <= M <= 16, 6 up to 32, 8 above), on Zipf(1.1)-skewed routing: slots of
    every size from one row to dozens take the VALU or the MFMA path side by
    side, every element against the oracle."""
    lay = moe_layer(0, wl=5, layer=300 + M, M=M, zipf_s=1.1)
    r, out = _run_block(m, gpu, lay)
    ids, w = oracle.route_topk(lay.logits, lay.k, lay.bias)
    check_routing_exact(r, ids, w, lay.E)
    counts = np.bincount(ids.ravel(), minlength=lay.E)
    assert counts.max() >= 3  # at least one MFMA slot at the default threshold
    ref = oracle.moe_block(lay.x, ids, w, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, None)
    assert tol_ratio(out, ref) <= 1.0


def test_moe_block_deterministic_and_workspace_reuse(m, gpu):
    """Repeated calls on one workspace, whatever it held before (it is filled
    with garbage first), give bit-identical outputs, in both schedules."""
    lay = moe_layer(seed=3, wl=202, M=16, E_=32, H_=512, I_=256, k=8, shared=True)
    d = upload_layer(lay, gpu, m)
    r = m.moe_route_topk(d["logits"], lay.k)
    WS_SHAPE = (16, 32, 8, 512, 256, True)
    ws = m.moe_workspace(*WS_SHAPE, gpu)
    ws.fill_(0xA5)
    call = lambda s: m.moe_nvfp4_decode(d["x"], r, d["gu"], d["dn"], d["sgu"], d["sdn"],
                                        workspace=ws, schedule=s, dense_min_rows=17)
    for s in (2, 3):
        a = call(s)
        outs = [call(s) for _ in range(4)]
        torch.cuda.synchronize()
        for b in outs:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))

