"""GPU parity of the router projection + top-k entry point against the oracle,
through the C ABI. Logits: |gpu - ref| <= 1e-2 |ref| + 1e-3 against the
oracle's float64 x W_r^T (bit for bit where the FP32 sums are exact).
Selection and grouping: bit for bit against the oracle's routing of the
GPU's own FP32 logits (near-ties of the float64 logits may order differently
after FP32 rounding; the logits are held to the tolerance instead)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import router_weights
from tests.helpers import check_routing_exact, routing_to_np, to_dev_bf16, tol_ratio

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(gpu):
    import nvfp4_moe_skinny_amd as m
    return m


def _bias(E, on, seed=0):
    return synth.normal_f32(synth.key(seed, 111, E), (E,), 0.0, 0.5) if on else None


@pytest.mark.parametrize("M,E,k,H,bias", [(1, 256, 8, 2048, False), (4, 256, 8, 2048, False),
                                          (9, 256, 8, 2048, False), (16, 256, 8, 2048, True),
                                          (64, 256, 8, 2048, True), (65, 256, 8, 2048, False),
                                          (256, 256, 8, 2048, False), (5, 64, 4, 512, False),
                                          (3, 128, 6, 1024, True), (7, 256, 8, 4096, False),
                                          (2, 100, 3, 2048, False), (1024, 256, 8, 2048, True)])
def test_route_project_parity(m, gpu, M, E, k, H, bias):
    x = synth.normal_bf16(synth.key(M, 110, E, H), (M, H))
    wr = router_weights(seed=M, wl=9, E_=E, H_=H)
    b = _bias(E, bias, M)
    bd = None if b is None else torch.from_numpy(b).to(gpu)
    logits, r = m.moe_route_project_topk(to_dev_bf16(x, gpu), to_dev_bf16(wr, gpu), k, bd)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    ref = oracle.router_logits(x, wr)
    assert tol_ratio(lg.astype(np.float64), ref) <= 1.0
    ids, w = oracle.route_topk(lg, k, b)
    g = check_routing_exact(r, ids, w, E)
    # the same as routing the logits through moe_route_topk
    r2 = m.moe_route_topk(logits, k, bd)
    torch.cuda.synchronize()
    g2 = routing_to_np(r2)
    for key in g:
        assert np.array_equal(g[key].view(np.uint32), g2[key].view(np.uint32)), key


@pytest.mark.parametrize("H", [512, 1024, 2048, 4096])
def test_route_project_exact_integer_logits(m, gpu, H):
    """Small-integer x and W_r: every FP32 partial sum is an integer below
    2^24, so the logits must equal the oracle's exactly (any wrong column,
    row or batch index shows)."""
    M, E, k = 11, 256, 8
    rng = np.random.default_rng(H)
    ints = np.array([0x0000, 0x3F80, 0x4000, 0x4040, 0xBF80, 0xC000], np.uint16)  # 0,1,2,3,-1,-2
    x = rng.choice(ints, (M, H)).astype(np.uint16)
    wr = rng.choice(ints, (E, H)).astype(np.uint16)
    logits, r = m.moe_route_project_topk(to_dev_bf16(x, gpu), to_dev_bf16(wr, gpu), k)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    ref = oracle.router_logits(x, wr)
    assert (lg.astype(np.float64) == ref).all()
    ids, w = oracle.route_topk(lg, k)
    check_routing_exact(r, ids, w, E)
