"""HIP-graph capture of the decode step (route + MoE decode): every replay must
reproduce the eager outputs bit for bit, with eager work and synchronisation
between replays."""
import numpy as np
import pytest
import torch

from synth.workloads import dense_skinny, moe_layer
from tests.helpers import pack, upload_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(gpu):
    import nvfp4_moe_skinny_amd as m
    return m


@pytest.mark.parametrize("M,shared,schedule", [(16, True, 2),
                                               (4, False, 2), (4, False, 3), (8, True, 3),
                                               (4, False, "fused"), (8, True, "fused"),
                                               (8, True, "fused+proj")])
def test_graph_replay_matches_eager(m, gpu, M, shared, schedule):
    lays = [moe_layer(seed=s, wl=400, layer=s, M=M, E_=64, H_=2048, I_=512, k=8, bias=shared,
                      shared=shared) for s in range(3)]
    devs = [upload_layer(l, gpu, m) for l in lays]
    WS_SHAPE = (M, 64, 8, 2048, 512, shared)
    ws = m.moe_workspace(*WS_SHAPE, gpu)
    routes = [m.routing_buffers(M, 64, 8, gpu) for _ in lays]
    outs = [torch.empty((M, 2048), dtype=torch.bfloat16, device=gpu) for _ in lays]
    # "fused+proj": a 2048 -> 64 projection of x computed in the down launch
    pws = [pack(dense_skinny(seed=s, M=M, K=2048, N=64, g=2.0 ** -9)[1], gpu, m) for s in range(3)]
    projs = [torch.empty((M, 64), dtype=torch.bfloat16, device=gpu) for _ in lays]

    def step(i):
        d = devs[i]
        if schedule in ("fused", "fused+proj"):  # routing inside the decode call
            pj = dict(proj=pws[i], proj_out=projs[i]) if schedule == "fused+proj" else {}
            m.moe_nvfp4_route_decode(d["x"], d["logits"], 8, d["gu"], d["dn"], d["bias"], d["sgu"],
                                     d["sdn"], residual=d["x"], workspace=ws, out=outs[i],
                                     ids=routes[i].ids, w=routes[i].w, **pj)
            return
        r = m.moe_route_topk(d["logits"], 8, d["bias"], out=routes[i])
        m.moe_nvfp4_decode(d["x"], r, d["gu"], d["dn"], d["sgu"], d["sdn"], residual=d["x"],
                           workspace=ws, out=outs[i], schedule=schedule)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    eager_p = [q.clone() for q in projs]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(3):
                step(i)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs + projs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e.view(torch.int16), o.view(torch.int16)), rep
        if schedule == "fused+proj":
            for e, q in zip(eager_p, projs):
                assert torch.equal(e.view(torch.int16), q.view(torch.int16)), rep
        step(rep % 3)  # eager work between replays
        torch.cuda.synchronize()
