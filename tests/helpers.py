"""Shared helpers for the GPU parity tests: upload canonical tensors, pack them
with the library, and compare against the oracle under the output tolerance
|gpu - ref| <= 1e-2 |ref| + 1e-3."""
import numpy as np
import torch

RTOL, ATOL = 1e-2, 1e-3


def bf16_bits_to_f64(bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(dev)


def dev_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def tol_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / (RTOL |ref| + ATOL); must be <= 1."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.isfinite(got).all():
        return float("inf")
    return float(np.max(np.abs(got - ref) / (RTOL * np.abs(ref) + ATOL)))


def pack(nv, dev, m):
    """synth.workloads.NVFP4 -> PackedNVFP4 on dev (m = the binding module)."""
    codes = torch.from_numpy(np.ascontiguousarray(nv.codes)).to(dev)
    scales = torch.from_numpy(np.ascontiguousarray(nv.scales)).to(dev)
    g = torch.from_numpy(np.ascontiguousarray(nv.g, dtype=np.float32)).to(dev)
    return m.nvfp4_pack(codes, scales, g)


def upload_layer(lay, dev, m):
    """MoELayer -> dict of device tensors and packed weights."""
    d = {
        "x": to_dev_bf16(lay.x, dev),
        "logits": torch.from_numpy(np.ascontiguousarray(lay.logits)).to(dev),
        "bias": None if lay.bias is None else torch.from_numpy(lay.bias).to(dev),
        "gu": pack(lay.gate_up, dev, m),
        "dn": pack(lay.down, dev, m),
        "sgu": None if lay.shared_gate_up is None else pack(lay.shared_gate_up, dev, m),
        "sdn": None if lay.shared_down is None else pack(lay.shared_down, dev, m),
    }
    return d


def routing_to_np(r):
    return {k: getattr(r, k).cpu().numpy() for k in
            ("ids", "w", "counts", "offsets", "pairs", "active", "active_offsets", "n_active")}


def check_routing_exact(r, ids_ref, w_ref, E):
    """Bit-exact ids / grouping, weights within 1e-6 (routing contract)."""
    import oracle
    g = routing_to_np(r)
    assert (g["ids"] == ids_ref).all(), "routing ids differ"
    counts, offsets, pairs, active, active_offsets, na = oracle.group_by_expert(ids_ref, E)
    assert (g["counts"] == counts).all()
    assert (g["active_offsets"] == active_offsets).all()
    assert (g["offsets"] == offsets).all()
    assert (g["pairs"] == pairs).all()
    assert (g["active"] == active).all()
    assert int(g["n_active"][0]) == na
    assert np.max(np.abs(g["w"].astype(np.float64) - w_ref)) <= 1e-6
    return g
