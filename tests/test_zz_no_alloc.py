"""moe_nvfp4_route_decode_static (h rows in the library's static device
array, no workspace) against moe_nvfp4_route_decode (caller's workspace):
bit-identical outputs, ids and weights on two calls in a row, the second
with a smaller input, both within tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from synth.workloads import moe_layer
from tests.helpers import dev_bf16_to_f64, to_dev_bf16, tol_ratio, upload_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(gpu):
    import nvfp4_moe_skinny_amd as m
    return m


def _both(m, gpu, lay, residual):
    d = upload_layer(lay, gpu, m)
    res = None if residual is None else to_dev_bf16(residual, gpu)
    M, k, H = lay.M, lay.k, lay.H
    outs = []
    for static in (False, True):
        out = torch.full((M, H), 3, dtype=torch.int16, device=gpu).view(torch.bfloat16)
        ids = torch.full((M, k), -7, dtype=torch.int32, device=gpu)
        w = torch.full((M, k), -1.0, dtype=torch.float32, device=gpu)
        m.moe_nvfp4_route_decode(d["x"], d["logits"], k, d["gu"], d["dn"], d["bias"], d["sgu"],
                                 d["sdn"], residual=res, out=out, ids=ids, w=w,
                                 static_scratch=static)
        outs.append((out, ids, w))
    torch.cuda.synchronize()
    (o0, i0, w0), (o1, i1, w1) = outs
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(i0, i1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    ids_ref, w_ref = oracle.route_topk(lay.logits, k, lay.bias)
    assert (i1.cpu().numpy() == ids_ref).all()
    ref = oracle.moe_block(lay.x, ids_ref, w_ref, lay.gate_up, lay.down, lay.shared_gate_up,
                           lay.shared_down, residual)
    assert tol_ratio(dev_bf16_to_f64(o1), ref) <= 1.0


def test_static_scratch_two_calls_second_smaller(m, gpu):
    # first call: 8 rows, shared expert, residual (72 h rows); second: 2 rows, none
    big = moe_layer(seed=11, wl=600, M=8, E_=64, H_=2048, I_=512, k=8, bias=True, shared=True)
    _both(m, gpu, big, big.x.copy())
    small = moe_layer(seed=12, wl=601, M=2, E_=32, H_=1024, I_=256, k=4)
    _both(m, gpu, small, None)


def test_static_scratch_rejects_oversized_calls(m, gpu):
    # (M*k + M) * I * 4 bytes of h rows beyond 4 MiB: refused before any launch
    a = m.MoeArgs()
    for f in ("x", "ids", "w", "w_gate_up", "w_down", "out"):
        setattr(a, f, 4096)
    a.M, a.E, a.k, a.H, a.I = 200, 256, 8, 2048, 1024
    a.dense_min_rows = 1 << 20
    st = m.lib.moe_nvfp4_route_decode_static(ctypes.byref(a), 4096, None, None)
    assert st == m.NVFP4MOE_ERR_UNSUPPORTED
    assert "scratch" in m.last_error_detail()
