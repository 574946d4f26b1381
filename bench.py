#!/usr/bin/env python3
"""Benchmark of the NVFP4 MoE decode step on one MI355X.

A step is one pass of the routed MoE hot path over one batch of rows: router
top-k, then gate_up -> SiLU*up -> down -> combine. For M <= 8 that is one
moe_nvfp4_route_decode call (routing folded into the gate_up launch); above,
moe_route_topk (top-k + grouping) then moe_nvfp4_decode. The headline workload
is one MoE block at M = 4 rows (one token plus three draft tokens verified
together): 256 experts, top-8, hidden 2048, expert width 512, NVFP4 weights,
BF16 activations.

To keep the 256 MB Infinity Cache from serving weights, each step uses the
next of `copies` independently seeded weight sets (>= 1 GB streams between two
uses of the same bytes) and the next of 64 router-logit sets. Inputs are
resident in HBM before timing starts. Steps are captured into a HIP graph and
replayed; `value` is algorithmic bytes per step (touched expert codes + scales
+ tensor scales, activations in and out, logits and routing arrays) over the
step time. For the roofline entry the decode call is timed on the stream it
runs on: over the graph replays when the call is the whole step (M <= 8),
else on its own with HIP events.

Every graph-timed workload runs at least one second of warm-up replays, then
five runs of at least 200 steps each (more when --steps asks for more), with
an event between runs; the line reports the median, mean and spread of the
runs. After timing, one output set the timed replays wrote is checked against
the float64 oracle: routing bit for bit, outputs within |gpu - ref| <=
1e-2 |ref| + 1e-3; the worst ratio goes in the line (parity_max_ratio) and
bench exits non-zero if it is above 1. The same byte count is read by the
read-ceiling kernel (one pass of 16-byte loads and nothing else) in the same
run, so the step is also reported against what a bare read of its bytes
takes on this chip.

The oracle (float64 C++ on the host) is timed on a bounded sample of the same
steps as a reported CPU baseline, single-threaded and with the host's threads.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 MoE decode achieved HBM GB/s (% of peak) + token-rows/s at M=4"
HBM_PEAK_GBS = 8000.0
CPU_LAYERS = 12  # weight copies kept on the host for the CPU-baseline sample
RTOL, ATOL = 1e-2, 1e-3  # the output tolerance against the float64 oracle
MIN_RUNS, MIN_RUN_STEPS, MIN_WARM_S = 5, 200, 1.0


# ---- host-side helpers (upload, compare) --------------------------------------------

def to_dev_bf16(bits, dev):
    """BF16 bit patterns (uint16 ndarray) -> torch bfloat16 on dev."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(dev)


def pack(nv, dev, m):
    """Canonical NVFP4 (codes, scales, g ndarrays) -> the library's packed layout on dev."""
    import torch
    codes = torch.from_numpy(np.ascontiguousarray(nv.codes)).to(dev)
    scales = torch.from_numpy(np.ascontiguousarray(nv.scales)).to(dev)
    g = torch.from_numpy(np.ascontiguousarray(nv.g, dtype=np.float32)).to(dev)
    return m.nvfp4_pack(codes, scales, g)


def dev_bf16_to_f64(t):
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def tol_ratio(got, ref):
    """max |got - ref| / (RTOL |ref| + ATOL): <= 1 passes."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if not np.isfinite(got).all():
        return float("inf")
    return float(np.max(np.abs(got - ref) / (RTOL * np.abs(ref) + ATOL)))


def host_info():
    """The machine the line was measured on: GPU, its compute units, the HIP
    runtime, the compiler the library was built with (recorded by the build:
    no child process is started here, so none runs under a profiler's
    preloaded library) and the host CPU the oracle baseline ran on."""
    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count,
            "hbm_bytes": props.total_memory, "torch": torch.__version__,
            "hip_runtime": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as fh:
            info["rocm"] = fh.read().strip()
    except OSError:
        pass
    try:
        with open(os.path.join(ROOT, "nvfp4_moe_skinny_amd", "libnvfp4moe.compiler.txt")) as fh:
            info["hipcc"] = fh.read().strip()[:200]
    except OSError:
        pass
    info.update(cpu_info())
    return info


def cpu_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "host_cpus_usable": usable}


# ---- timing ----------------------------------------------------------------------------

def capture(step, S):
    """A HIP graph of step(0 .. S-1), captured on a side stream."""
    import torch
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(S):
                step(i)
    torch.cuda.synchronize()
    return graph


def replay_timed(graph, S, want_steps, min_run_steps=MIN_RUN_STEPS):
    """Warm-up replays for at least MIN_WARM_S seconds, then MIN_RUNS runs of
    at least max(min_run_steps, want_steps / MIN_RUNS) steps each (whole
    replays of the S-step graph), an event between runs. Returns (ms per
    step over all runs, steps timed, per-run stats)."""
    import torch
    t0 = time.time()
    warm = 0
    while time.time() - t0 < MIN_WARM_S or warm < 2:
        graph.replay()
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per_run = max(min_run_steps, int(np.ceil(want_steps / MIN_RUNS)))
    reps = max(1, int(np.ceil(per_run / S)))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(MIN_RUNS + 1)]
    evs[0].record()
    for r in range(MIN_RUNS):
        for _ in range(reps):
            graph.replay()
        evs[r + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[r].elapsed_time(evs[r + 1]) / (reps * S) for r in range(MIN_RUNS)])
    stats = {"n": MIN_RUNS, "steps_per_run": reps * S, "warmup_replays": warm,
             "warmup_s": round(time.time() - t0, 2),
             "median_ms_per_step": round(float(np.median(per)), 6),
             "mean_ms_per_step": round(float(per.mean()), 6),
             "std_ms_per_step": round(float(per.std(ddof=1)), 6)}
    return evs[0].elapsed_time(evs[-1]) / (MIN_RUNS * reps * S), MIN_RUNS * reps * S, stats


def read_ceiling(nbytes, m, want_steps=4000):
    """Time of one bare read of nbytes (nvfp4moe_stream_read: the 16-byte
    nontemporal loads the weight streams use, nothing computed), over
    distinct buffers cycled through >= 2 GB so every pass reads HBM."""
    import torch
    nbytes = max(16, int(nbytes) // 16 * 16)
    copies = max(2, int(np.ceil(2e9 / nbytes)))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sinks = [torch.empty(m.nvfp4moe_stream_blocks(nbytes), dtype=torch.int32, device="cuda")
             for _ in range(copies)]

    def step(i):
        m.nvfp4moe_stream_read(bufs[i % copies], sink=sinks[i % copies])

    for i in range(copies):
        step(i)
    graph = capture(step, copies * int(np.ceil(16 / copies)))
    ms, _, _ = replay_timed(graph, copies * int(np.ceil(16 / copies)),
                            min(want_steps, 2000 if nbytes < 5e8 else 50),
                            min_run_steps=min(MIN_RUN_STEPS, 20 if nbytes > 5e8 else 200))
    del graph, bufs, sinks
    torch.cuda.empty_cache()
    return ms * 1e3


# the device code of one moe_nvfp4_decode call (all of its launches)
DECODE_SOURCES = ("common.hpp", "tile.hpp", "dense.hpp", "moe.hpp", "staged.hpp", "route.hpp",
                  "fused.hpp", "api.hip")


def kernel_source_hash():
    """Hash of the decode call's kernel sources, to tie recorded counters to the
    code: comments and whitespace are left out, so that a comment edit does
    not void them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_moe_skinny_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per decode call (its gate_up, down and combine launches) from
    the committed FETCH_SIZE/WRITE_SIZE summary of this workload, or None if
    there is none or the kernels have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_counters.md")
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_hash: ")))
    except OSError:
        return None
    if fields.get("source_hash", "").strip() != kernel_source_hash():
        return None
    return float(fields["traffic_bytes_per_launch"])


def expert_bytes(H, I):
    """Canonical NVFP4 bytes of one expert: gate_up [2I][H] + down [H][I]
    (codes + E4M3 scales + FP32 tensor scale)."""
    gu = 2 * I * H // 2 + 2 * I * H // 16 + 4
    dn = H * I // 2 + H * I // 16 + 4
    return gu + dn


def step_bytes(M, E, k, H, I, n_active, shared, bias, grouped=True):
    b = n_active * expert_bytes(H, I) + (expert_bytes(H, I) if shared else 0)
    b += M * H * 2 * 2          # x in, out
    b += M * E * 4              # logits
    b += E * 4 if bias else 0   # logit bias
    b += M * k * (4 + 4) * 2    # ids, w written then read
    if grouped:                 # counts, offsets, active, n_active, pairs
        b += (E + E + 1 + E + 1) * 4 + M * k * 4 * 2
    return b


def decode_kernels(schedule, M):
    """The launches of one decode call under the library's schedule choice."""
    gate = "staged_gate_split_kernel" if M <= 16 else "staged_gate_kernel"
    if schedule == 3 or (schedule == 0 and M <= 8):
        return f"moe_nvfp4_decode (one call: {gate}, token_down_combine_kernel)"
    return f"moe_nvfp4_decode (one call: {gate}, staged_down_kernel, staged_combine_kernel)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="m4",
                   choices=["m4", "m16", "m256", "dense", "head32k", "head248k", "fp8qkv",
                            "fp8o", "router", "quant", "stack40", "ceiling"])
    p.add_argument("--rows", type=int, default=0, help="rows M of a skinny-GEMM workload")
    p.add_argument("--dense-min-rows", type=int, default=0,
                   help="rows from which a slot uses MFMA (0 = library default)")
    p.add_argument("--schedule", type=int, default=0, choices=[0, 2, 3],
                   help="0 = library choice, 2 = three launches, 3 = two launches")
    p.add_argument("--path", default="auto", choices=["auto", "separate", "fused"],
                   help="separate: moe_route_topk + moe_nvfp4_decode; fused: "
                        "moe_nvfp4_route_decode (few rows); auto: fused for M <= 8")
    p.add_argument("--copies", type=int, default=0, help="weight sets cycled (0: >= 1 GB)")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="oracle time budget per thread count (single-threaded, then all threads)")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the read-ceiling pass at the step's byte count")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager-calls", type=int, default=400, help=">= 2")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="only run a plain device copy of this many MB (counter calibration)")
    return p.parse_args()


def calibrate_copy(mb):
    """A plain device-to-device copy of known size: reading FETCH_SIZE and
    WRITE_SIZE for it under rocprofv3 gives the counters' scale factor."""
    import torch
    n = mb * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "copies": 5}), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU's share of a sharded model)", file=sys.stderr)
        return 2
    if args.calibrate_copy_mb:
        return calibrate_copy(args.calibrate_copy_mb)
    if args.workload.startswith("head"):
        return bench_head(args)
    if args.workload == "dense":
        return bench_dense(args)
    if args.workload.startswith("fp8"):
        return bench_fp8(args)
    if args.workload == "router":
        return bench_router(args)
    if args.workload == "quant":
        return bench_quant(args)
    if args.workload == "stack40":
        return bench_stack(args)
    if args.workload == "ceiling":
        return bench_ceiling(args)
    import torch

    import nvfp4_moe_skinny_amd as m
    from synth import workloads as W

    dev = torch.device("cuda:0")
    zipf = None
    if args.workload == "m4":
        make = lambda c: W.moe_layer(0, wl=2, layer=c, M=4)
        name = "moe_block_m4_e256_top8_h2048_i512"
        wl, touched = 2, 31
    elif args.workload == "m16":
        make = lambda c: W.moe_layer(0, wl=3, layer=c, M=16, bias=True, shared=True)
        name = "moe_block_m16_e256_top8_h2048_i512_bias_shared"
        wl, touched = 3, 84
    else:
        zipf = 1.1
        make = lambda c: W.moe_layer(0, wl=5, layer=c, M=256, zipf_s=zipf)
        name = "moe_block_m256_e256_top8_h2048_i512_zipf1.1"
        wl, touched = 5, 229
    lay0 = make(0)
    M, E, k, H, I = lay0.M, lay0.E, lay0.k, lay0.H, lay0.I
    shared = lay0.shared_gate_up is not None
    bias = lay0.bias is not None
    per_step_est = touched * expert_bytes(H, I)
    copies = args.copies or int(np.ceil(1e9 / per_step_est)) + 1

    # ---- resident inputs -------------------------------------------------------------
    t0 = time.time()
    weights = []
    layers_host = []
    for c in range(copies):
        lay = lay0 if c == 0 else make(c)
        gu, dn = pack(lay.gate_up, dev, m), pack(lay.down, dev, m)
        sgu = pack(lay.shared_gate_up, dev, m) if shared else None
        sdn = pack(lay.shared_down, dev, m) if shared else None
        weights.append((gu, dn, sgu, sdn))
        if c < CPU_LAYERS:
            layers_host.append(lay)
        torch.cuda.synchronize()
    # 64 router-logit / activation sets (small tensors: only the logits and x are used)
    n_sets = 64
    logit_sets = [W.moe_layer(0, wl=wl, layer=1000 + i, M=M, E_=E, H_=32, I_=32, k=k, bias=bias,
                              zipf_s=zipf) for i in range(n_sets)]
    x_host = [W.normal_bf16(W.key(0, wl, 1000 + i, W.T_X, 1), (M, H)) for i in range(n_sets)]
    xs = [to_dev_bf16(xh, dev) for xh in x_host]
    lg = [torch.from_numpy(L.logits).to(dev) for L in logit_sets]
    bs = [torch.from_numpy(L.bias).to(dev) if bias else None for L in logit_sets]
    routes = [m.routing_buffers(M, E, k, dev) for _ in range(n_sets)]
    outs = [torch.empty((M, H), dtype=torch.bfloat16, device=dev) for _ in range(n_sets)]
    ws = m.moe_workspace(M, E, k, H, I, shared, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    fused = args.path == "fused" or (args.path == "auto" and args.schedule == 0 and M <= 8)

    # one decode call: routed experts + shared + combine (fused: with the routing)
    def decode_call(i):
        c, j = i % copies, i % n_sets
        gu, dn, sgu, sdn = weights[c]
        if fused:
            m.moe_nvfp4_route_decode(xs[j], lg[j], k, gu, dn, bs[j], sgu, sdn, workspace=ws,
                                     out=outs[j], ids=routes[j].ids, w=routes[j].w,
                                     dense_min_rows=args.dense_min_rows)
        else:
            m.moe_nvfp4_decode(xs[j], routes[j], gu, dn, sgu, sdn, workspace=ws, out=outs[j],
                               schedule=args.schedule, dense_min_rows=args.dense_min_rows)

    # one step of the hot path: (weight copy c, logits/x set j)
    def step(i):
        j = i % n_sets
        if not fused:
            m.moe_route_topk(lg[j], k, bs[j], out=routes[j])
        decode_call(i)

    # the graph holds S steps: step i uses weight copy i % copies and set i % n_sets
    S = copies * int(np.ceil(n_sets / copies))
    for i in range(max(args.warmup, S)):
        step(i)
    torch.cuda.synchronize()
    graph = capture(step, S)
    wall0 = time.time()
    ms_per_step, steps, runs = replay_timed(graph, S, args.steps)
    wall = time.time() - wall0

    # bytes from each step's actual routing (read back after the timed region)
    n_act = np.array([len(np.unique(routes[j].ids.cpu().numpy())) for j in range(n_sets)])
    bytes_per_set = np.array([step_bytes(M, E, k, H, I, int(na), shared, bias, not fused)
                              for na in n_act])
    mean_bytes = float(np.mean([bytes_per_set[i % n_sets] for i in range(S)]))
    gbs = mean_bytes / (ms_per_step * 1e-3) / 1e9
    rows_per_s = M / (ms_per_step * 1e-3)

    # parity of what the timed replays left in output set 0: the last step of
    # the graph that wrote it used weight copy c
    last = max(i for i in range(S) if i % n_sets == 0)
    c = last % copies
    lay_c = layers_host[c] if c < len(layers_host) else make(c)
    parity = check_parity(lay_c, logit_sets[0], x_host[0], routes[0], outs[0], fused, M, E, k)

    # eager: each decode call timed with events on its own stream (roofline entry)
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.eager_calls)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.eager_calls)]
    decode_bytes = []
    for i in range(args.eager_calls):
        j = i % n_sets
        if not fused:
            m.moe_route_topk(lg[j], k, bs[j], out=routes[j])
        starts[i].record(stream)
        decode_call(i)
        ends[i].record(stream)
        b = n_act[j] * expert_bytes(H, I) + (expert_bytes(H, I) if shared else 0) + M * H * 4
        if fused:  # logits (+ bias) in, ids and w out
            b += M * E * 4 + (E * 4 if bias else 0) + M * k * 8
        else:      # ids, w and the grouping arrays in
            b += M * k * 8 + (E + 1 + E + 1) * 4 + M * k * 4
        decode_bytes.append(b)
    torch.cuda.synchronize()
    skip = min(20, args.eager_calls // 2)  # warm calls only
    dec_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])[skip:]
    dec_bytes = float(np.mean(decode_bytes[skip:]))
    dec_avg_ms = float(dec_ms.mean())
    eager_call_us = dec_avg_ms * 1e3
    if fused:
        # the step is the one call: its duration over the timed region (graph
        # replay, events on the replay stream) and its algorithmic bytes
        dec_avg_ms, dec_bytes = ms_per_step, mean_bytes
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9

    # eager step rate (host launch included), for context
    torch.cuda.synchronize()
    e0 = time.time()
    for i in range(args.eager_calls):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.time() - e0) * 1e3 / args.eager_calls
    del graph

    outs_ok = all(torch.isfinite(o.float()).all().item() for o in outs)
    ceiling = None
    if not args.no_ceiling:
        del weights
        torch.cuda.empty_cache()
        c_us = read_ceiling(mean_bytes, m)
        ceiling = {"bytes": round(mean_bytes), "us": round(c_us, 3),
                   "GB/s": round(mean_bytes / (c_us * 1e-6) / 1e9, 1),
                   "step_frac_of_ceiling": round(c_us / (ms_per_step * 1e3), 4),
                   "kernel": "nvfp4moe_stream_read, one launch, buffers cycled over >= 2 GB"}

    record = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "M": M, "E": E, "top_k": k, "hidden": H,
                   "expert_inter": I, "weights": "nvfp4 e2m1 + e4m3/16 + f32",
                   "accumulate": "f32", "shared_expert": shared, "logit_bias": bias,
                   "weight_copies": copies, "logit_sets": n_sets, "graph_steps": S,
                   "timing": "hip graph replay, events",
                   "schedule": args.schedule, "dense_min_rows": args.dense_min_rows,
                   "path": "moe_nvfp4_route_decode" if fused
                           else "moe_route_topk + moe_nvfp4_decode"},
        "rows_per_s": round(rows_per_s, 1),
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "runs": runs,
        "bytes_per_step": round(mean_bytes),
        "touched_experts_mean": float(np.mean(n_act)),
        "eager_ms_per_step": round(eager_ms, 4),
        "roofline": {"bound": "hbm",
                     "kernel": ("moe_nvfp4_route_decode (one call: fused_route_gate_kernel, "
                                "token_down_combine_kernel)" if fused
                                else decode_kernels(args.schedule, M)),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"moe_decode_{args.workload}"),
                     "avg_launch_us": round(dec_avg_ms * 1e3, 3),
                     "bytes_per_launch": round(dec_bytes),
                     "timing": ("the call's duration over the timed graph replays" if fused
                                else "eager calls, events on the launching stream"),
                     "eager_call_us": round(eager_call_us, 3)},
        "read_ceiling": ceiling,
        "parity": parity, "parity_max_ratio": parity["max_ratio"],
        "outputs_finite": outs_ok, "setup_s": round(setup_s, 1), "wall_s": round(wall, 3),
        "host": host_info(),
    }
    failed = (not outs_ok or gbs <= 0 or not np.isfinite(gbs) or not parity["ok"])
    if failed:
        print(json.dumps(record), flush=True)
        print("bench: invalid result (parity or non-finite outputs)", file=sys.stderr)
        return 1

    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(layers_host, logit_sets, x_host, copies, n_sets,
                                              args.cpu_seconds, shared, bias)
    print(json.dumps(record), flush=True)
    return 0


def check_parity(lay, lset, x_host, route, out, fused, M, E, k):
    """Routing and outputs of one timed step against the oracle: ids (and,
    without the fused path, the grouping) bit for bit, weights within 1e-6,
    outputs within the output tolerance."""
    import oracle
    ids, w = oracle.route_topk(lset.logits, k, lset.bias)
    got_ids = route.ids.cpu().numpy()
    ids_ok = bool((got_ids == ids).all())
    w_err = float(np.max(np.abs(route.w.cpu().numpy().astype(np.float64) - w)))
    group_ok = True
    if not fused:
        counts, offsets, pairs, active, active_offsets, na = oracle.group_by_expert(ids, E)
        group_ok = bool((route.pairs.cpu().numpy() == pairs).all() and
                        (route.active_offsets.cpu().numpy() == active_offsets).all() and
                        int(route.n_active.cpu().numpy()[0]) == na)
    lay_x = type(lay)(**{**lay.__dict__, "x": x_host, "M": M})
    ref = oracle.moe_block_touched(lay_x, ids, w)
    ratio = tol_ratio(dev_bf16_to_f64(out), ref)
    ok = ids_ok and group_ok and w_err <= 1e-6 and ratio <= 1.0
    return {"ok": ok, "max_ratio": round(ratio, 4), "ids_exact": ids_ok, "grouping_exact": group_ok,
            "w_max_abs_err": w_err, "checked": "output set 0 as the timed replays left it",
            "oracle_threads": oracle.threads()}


def time_graph(step, copies, args, min_run_steps=MIN_RUN_STEPS):
    """Captures S = a multiple of copies (>= 16) calls step(0 .. S-1) in one
    HIP graph and times its replays (replay_timed): (ms per call, calls
    timed); the runs' spread is kept for the JSON line (run_stats)."""
    import torch
    S = copies * int(np.ceil(16 / copies))
    for i in range(max(args.warmup, S)):
        step(i)
    torch.cuda.synchronize()
    graph = capture(step, S)
    ms, n, stats = replay_timed(graph, S, args.steps, min_run_steps)
    _RUNS.clear()
    _RUNS.update(stats)
    return ms, n


_RUNS = {}


def run_stats():
    """The per-run spread of the last time_graph call."""
    return dict(_RUNS)


def bench_fp8(args):
    """FP8 E4M3 skinny product with one tensor scale (attention projections):
    M rows (default 4) times [N][K] FP8 weights, K = 2048 -> N = 5120 (fp8qkv)
    or K = 4096 -> N = 2048 (fp8o). The weights are one seeded matrix copied
    to enough device buffers (>= 1 GB in all) that replays read HBM, not the
    last-level cache. Not the headline line."""
    import torch

    import nvfp4_moe_skinny_amd as m
    from synth import workloads as W

    dev = torch.device("cuda:0")
    K, N = (2048, 5120) if args.workload == "fp8qkv" else (4096, 2048)
    M = args.rows or 4
    x, w, s = W.fp8_projection(seed=0, M=M, K=K, N=N)
    copies = args.copies or int(np.ceil(1e9 / w.nbytes)) + 1
    wd = torch.from_numpy(w).to(dev)
    ws = [wd.clone() for _ in range(copies)]
    xd = to_dev_bf16(x, dev)
    sc = torch.tensor([s], dtype=torch.float32, device=dev)
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    def step(i):
        m.fp8_skinny_gemm(xd, ws[i % copies], sc, out=outs[i % copies])

    ms, n_steps = time_graph(step, copies, args)
    import oracle
    ratio = tol_ratio(dev_bf16_to_f64(outs[0]), oracle.gemm_fp8(x, w, s))
    step_bytes = w.nbytes + 4 + M * K * 2 + M * N * 2
    gbs = step_bytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "FP8 skinny GEMM achieved HBM GB/s (attention projection)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"fp8_skinny_gemm_m{M}_k{K}_n{N}", "M": M, "K": K, "N": N,
                   "weights": "fp8 e4m3 + one f32 tensor scale", "weight_copies": copies,
                   "timing": "hip graph replay, events"},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_bytes,
        "runs": run_stats(), "parity_max_ratio": round(ratio, 4),
    }), flush=True)
    return 0 if ratio <= 1.0 else 1


def bench_router(args):
    """Router projection + top-k + grouping (moe_route_project_topk): M rows
    (default 4) of BF16 x [M][2048] times a BF16 router [256][2048], k = 8.
    Router copies cycled so the 1 MB matrix comes from HBM. Not the headline."""
    import torch

    import nvfp4_moe_skinny_amd as m
    from synth import workloads as W

    dev = torch.device("cuda:0")
    M, E, H, k = args.rows or 4, 256, 2048, 8
    x = to_dev_bf16(W.normal_bf16(W.key(0, 9, 0, W.T_X, 0), (M, H)), dev)
    wr = to_dev_bf16(W.router_weights(seed=0, wl=9), dev)
    copies = args.copies or 300
    wrs = [wr.clone() for _ in range(copies)]
    bufs = [m.routing_buffers(M, E, k, dev) for _ in range(copies)]
    logits = [torch.empty((M, E), dtype=torch.float32, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    def step(i):
        j = i % copies
        m.moe_route_project_topk(x, wrs[j], k, out=bufs[j], logits=logits[j])

    ms, n_steps = time_graph(step, copies, args)
    step_bytes = E * H * 2 + M * H * 2 + M * E * 4 * 2 + M * k * 8
    print(json.dumps({
        "metric": "router projection + top-k latency", "value": round(ms * 1e3, 3),
        "unit": "us", "n_gpus": 1, "steps": n_steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"route_project_m{M}_e{E}_h{H}_k{k}", "M": M, "E": E, "H": H,
                   "top_k": k, "router_copies": copies, "timing": "hip graph replay, events"},
        "achieved_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 2), "bytes_per_step": step_bytes,
        "runs": run_stats(),
    }), flush=True)
    return 0


def bench_quant(args):
    """Device quantizer (nvfp4_quantize) over one layer's gate_up expert set,
    BF16 [256][1024][2048] (1 GiB in, 0.28 GiB out). 32 seeded matrices are
    generated on the host and tiled to 256 on the device. Not the headline."""
    import torch

    import nvfp4_moe_skinny_amd as m
    from synth import workloads as W

    dev = torch.device("cuda:0")
    G, N, K = 256, 1024, 2048
    base = to_dev_bf16(W.normal_bf16(W.key(0, 8, 0, W.T_X, 0), (32, N, K), 0.0, 0.02), dev)
    x = base.repeat(G // 32, 1, 1).contiguous()
    del base
    codes = torch.empty((G, N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((G, N, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(G, dtype=torch.float32, device=dev)
    L = m.lib
    ptrs = (x.data_ptr(), codes.data_ptr(), scales.data_ptr(), g.data_ptr())

    def call():
        st = L.nvfp4_quantize(ptrs[0], G, N, K, ptrs[1], ptrs[2], ptrs[3],
                              torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"nvfp4_quantize: {st}")

    for _ in range(max(2, min(args.warmup, 5))):
        call()
    torch.cuda.synchronize()
    n = max(3, min(args.steps, 20))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(n):
        call()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / n
    step_bytes = G * N * K * 2 + G * N * (K // 2 + K // 16) + G * 4  # x once (two passes read it twice)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "NVFP4 quantizer achieved HBM GB/s", "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"nvfp4_quantize_g{G}_n{N}_k{K}", "G": G, "N": N, "K": K,
                   "timing": "eager launches, events"},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_bytes,
        "runs": run_stats(),
    }), flush=True)
    return 0


def bench_dense(args):
    """The single dense NVFP4 matrix: M = 1 BF16 row ~N(0,1) (--rows: M rows)
    times W [512][2048] (uniform codes, E4M3 scales 2^U[-4,4), g = 1.0),
    594,948 bytes a call at M = 1.
    Calls cycle through >= 2048 distinct seeded matrices (1.2 GB, copy 0 is
    the canonical seed-0 matrix) so that each reads HBM, not the last-level
    cache. value = the amortised rate of the calls in a graph; beside it the
    single-launch latency (each call alone between two events, eager). One
    such call is latency-bound by construction: its bytes stream in ~74 ns at
    8 TB/s, far below a launch's own cost."""
    import torch

    import nvfp4_moe_skinny_amd as m
    import oracle
    from synth import workloads as W

    dev = torch.device("cuda:0")
    M, K, N = args.rows or 1, 2048, 512
    copies = max(args.copies or 2048, 16)
    t0 = time.time()
    ws, xs, host = [], [], []
    for c in range(copies):
        x, w = W.dense_skinny(seed=0, M=M, layer=c)
        ws.append(pack(w, dev, m))
        xs.append(to_dev_bf16(x, dev))
        if c < 64:
            host.append((x, w))
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(i):
        m.nvfp4_skinny_gemm(xs[i % copies], ws[i % copies], out=outs[i % copies])

    ms, n_steps = time_graph(step, copies, args)
    runs = run_stats()
    # what the timed replays left in output 0 (written by copy 0's calls)
    x0, w0 = host[0]
    ratio = tol_ratio(dev_bf16_to_f64(outs[0]), oracle.gemm(x0, w0.codes[0], w0.scales[0],
                                                            float(w0.g[0])))
    # single launches: each call alone between two events on its stream
    stream = torch.cuda.current_stream()
    n_eager = max(args.eager_calls, 64)
    st = [torch.cuda.Event(enable_timing=True) for _ in range(n_eager)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(n_eager)]
    for i in range(n_eager):
        st[i].record(stream)
        step(i)
        en[i].record(stream)
        stream.synchronize()  # nothing queued behind: the call's own latency
    lat = np.array([a.elapsed_time(b) for a, b in zip(st, en)])[8:] * 1e3
    w_bytes = N * K // 2 + N * K // 16 + 4
    step_b = w_bytes + M * K * 2 + M * N * 2
    gbs = step_b / (ms * 1e-3) / 1e9
    ceiling_us = None if args.no_ceiling else read_ceiling(step_b, m)
    # the library's choice for K = 2048, N = 512 (4-16 rows: the split-K MFMA kernel)
    gemm_kernel = "skinny_gemm_kernel<64>" if M < 4 else (
        "skinny_gemm_splitk_kernel" if M <= 16 else "skinny_gemm_dense_kernel")
    record = {
        "metric": f"NVFP4 dense skinny GEMM achieved HBM GB/s (single 2048->512 matrix, M={M})",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"nvfp4_skinny_gemm_m{M}_k2048_n512", "M": M, "K": K, "N": N,
                   "g": 1.0, "distinct_matrices": copies,
                   "timing": "hip graph replay, events (amortised over the calls)"},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_b,
        "runs": runs,
        "single_launch_us": {"median": round(float(np.median(lat)), 3),
                             "mean": round(float(lat.mean()), 3),
                             "min": round(float(lat.min()), 3), "calls": int(lat.size),
                             "timing": "eager, each call alone between two events"},
        "roofline": {"bound": "hbm", "kernel": f"{gemm_kernel} (one launch a call)",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(ms * 1e3, 4), "bytes_per_launch": step_b,
                     "timing": "launches in a graph, amortised; latency-bound (74 ns of bytes)"},
        "read_ceiling": None if ceiling_us is None else
        {"bytes": step_b, "us": round(ceiling_us, 3),
         "step_frac_of_ceiling": round(ceiling_us / (ms * 1e3), 4)},
        "parity_max_ratio": round(ratio, 4), "setup_s": round(setup_s, 1),
        "host": host_info(),
    }
    if not np.isfinite(gbs) or ratio > 1.0:
        print(json.dumps(record), flush=True)
        print("bench: invalid result (parity)", file=sys.stderr)
        return 1
    if not args.no_cpu_baseline:
        def one(i):
            x, w = host[i % len(host)]
            oracle.gemm(x, w.codes[0], w.scales[0], float(w.g[0]))
            return step_b
        record["cpu_baseline"] = baseline_record(one, args.cpu_seconds, M,
                                                 "2048->512 products (one row each)")
    print(json.dumps(record), flush=True)
    return 0


def bench_head(args):
    """Large-N skinny GEMM: M = 6 rows times a [N][2048] NVFP4 head (N = 32768,
    the draft head; N = 248000, the full head). Not the headline line: a
    measurement of the same streaming product at a bandwidth-sized shape."""
    import torch

    import nvfp4_moe_skinny_amd as m
    from synth import workloads as W

    dev = torch.device("cuda:0")
    N = 32768 if args.workload == "head32k" else 248000
    M = args.rows or 6
    w_bytes = N * 2048 // 2 + N * 2048 // 16 + 4
    copies = args.copies or int(np.ceil(1e9 / w_bytes)) + 1
    ws, xs = [], []
    for c in range(copies):
        x, w = W.draft_head(seed=0, M=M, N=N, layer=c)
        ws.append(pack(w, dev, m))
        xs.append(to_dev_bf16(x, dev))
        if c == 0:
            x0, w0 = x, w
        torch.cuda.synchronize()
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]

    def step(i):
        m.nvfp4_skinny_gemm(xs[i % copies], ws[i % copies], out=outs[i % copies])

    ms, n_steps = time_graph(step, copies, args)
    import oracle  # what the timed replays left in output 0 (copy 0's calls)
    ratio = tol_ratio(dev_bf16_to_f64(outs[0]),
                      oracle.gemm(x0, w0.codes[0], w0.scales[0], float(w0.g[0])))
    step_bytes = w_bytes + M * 2048 * 2 + M * N * 2
    gbs = step_bytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "NVFP4 skinny GEMM achieved HBM GB/s (large-N head)", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": n_steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"nvfp4_skinny_gemm_m{M}_k2048_n{N}", "M": M, "K": 2048, "N": N,
                   "weight_copies": copies, "timing": "hip graph replay, events"},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_bytes,
        "runs": run_stats(), "parity_max_ratio": round(ratio, 4),
    }), flush=True)
    return 0 if ratio <= 1.0 else 1


def bench_stack(args):
    """Sustained weight streaming: the 40-block stack at M = 8 rows, all 40
    layers' weights resident (about 18 GB of packed experts, more than any
    cache, so no copies are cycled). One step runs the 40 layers back to back
    as a chain: per layer one moe_nvfp4_route_decode call (routing from the
    layer's synthetic logits, routed + shared experts, residual x_l) writing
    x_{l+1}, with the dense 2048->64 projection of x_l computed by blocks of
    its down launch. The step is captured in
    one HIP graph (at most 320 steps are timed); bytes are every layer's
    touched experts + the shared expert + the projection + activations, from
    the routing each layer actually took."""
    import torch

    import nvfp4_moe_skinny_amd as m
    from synth import workloads as W

    dev = torch.device("cuda:0")
    n_layers, M = W.STACK_LAYERS, W.STACK_M
    t0 = time.time()
    layers = []
    for l in range(n_layers):
        lay = W.stack_layer(l)
        layers.append((pack(lay.gate_up, dev, m), pack(lay.down, dev, m),
                       pack(lay.shared_gate_up, dev, m), pack(lay.shared_down, dev, m),
                       pack(lay.extra["proj"], dev, m), torch.from_numpy(lay.logits).to(dev)))
        torch.cuda.synchronize()
    E, k, H, I, N = lay.E, lay.k, lay.H, lay.I, W.STACK_PROJ_N
    resident = sum(sum(int(t.data.numel()) for t in L[:5]) for L in layers)
    xs = [to_dev_bf16(W.stack_x0(), dev)] + [torch.empty((M, H), dtype=torch.bfloat16, device=dev)
                                             for _ in range(n_layers)]
    projs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
    routes = [m.routing_buffers(M, E, k, dev) for _ in range(n_layers)]
    ws = m.moe_workspace(M, E, k, H, I, True, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # one call per layer: the projection's blocks ride in the block's down
    # launch (as its own launch it cost 4.3 us a layer; on a second stream,
    # joined per step, the layer measured slower still)
    def step(_i):
        for l in range(n_layers):
            gu, dn, sgu, sdn, pw, lg = layers[l]
            m.moe_nvfp4_route_decode(xs[l], lg, k, gu, dn, None, sgu, sdn, residual=xs[l],
                                     workspace=ws, out=xs[l + 1], ids=routes[l].ids,
                                     w=routes[l].w, proj=pw, proj_out=projs[l])

    args.steps = min(args.steps, 320)  # a step streams ~4 GB: keep the timed region short
    ms, n_steps = time_graph(step, 1, args)
    n_act = [len(np.unique(r.ids.cpu().numpy())) for r in routes]
    proj_bytes = N * H // 2 + N * H // 16 + 4 + M * N * 2
    step_b = sum(step_bytes(M, E, k, H, I, na, True, False, grouped=False) for na in n_act)
    step_b += n_layers * (proj_bytes + M * H * 2)  # + the projection, + the residual read
    gbs = step_b / (ms * 1e-3) / 1e9
    xf = xs[-1].float()
    ok = bool(torch.isfinite(xf).all().item())
    print(json.dumps({
        "metric": "NVFP4 MoE 40-layer stack achieved HBM GB/s (sustained weight streaming)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "moe_stack_40_layers_m8_e256_top8_h2048_i512_shared_proj64",
                   "layers": n_layers, "M": M, "E": E, "top_k": k, "hidden": H,
                   "expert_inter": I, "proj_n": N, "resident_weight_bytes": resident,
                   "timing": "hip graph replay of the 40-layer chain, events",
                   "path": "moe_nvfp4_route_decode (with the projection) per layer"},
        "rows_per_s": round(M / (ms * 1e-3), 1),
        "layer_us": round(ms * 1e3 / n_layers, 3),
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": step_b,
        "runs": run_stats(),
        "touched_experts_mean": float(np.mean(n_act)),
        "outputs_finite": ok, "setup_s": round(setup_s, 1),
    }), flush=True)
    return 0 if ok else 1


def bench_ceiling(args):
    """The read ceiling (nvfp4moe_stream_read: one pass of 16-byte nontemporal
    loads, the weight streams' kind): a 4 GiB buffer, and buffers of the M=4
    step's size (54 MB), of its two launches' weight bytes (36 MB gate_up,
    18 MB down: 30.6 experts), those two as back-to-back launches, and the
    M=16 step's (147 MB), each cycled over >= 2 GB of distinct buffers so that
    every pass reads HBM, in graphs timed with events. value = the 4 GiB
    rate."""
    import torch

    import nvfp4_moe_skinny_amd as m

    dev = torch.device("cuda:0")
    res = {}
    for name, nbytes in (("4GiB", 4 << 30), ("54MB", 54_117_108 // 16 * 16),
                         ("36MB", 36_097_351 // 16 * 16), ("18MB", 18_048_737 // 16 * 16),
                         ("147MB", 147_000_000 // 16 * 16)):
        copies = max(1, int(np.ceil(2e9 / nbytes)))
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        sinks = [torch.empty(m.nvfp4moe_stream_blocks(nbytes), dtype=torch.int32, device=dev)
                 for _ in range(copies)]

        def step(i, bufs=bufs, sinks=sinks, copies=copies):
            m.nvfp4moe_stream_read(bufs[i % copies], sink=sinks[i % copies])

        saved = args.steps
        args.steps = min(args.steps, 200 if nbytes > 1e9 else 4000)
        ms, n = time_graph(step, copies, args)
        args.steps = saved
        res[name] = {"bytes": nbytes, "us": round(ms * 1e3, 3),
                     "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "passes_timed": n,
                     "buffers_cycled": copies}
        del bufs, sinks
        torch.cuda.empty_cache()
    # two launches back to back, 36 MB then 18 MB: the M=4 step's shape (gate_up
    # weights, then down weights) with nothing computed and nothing waited for
    sizes = (36_097_351 // 16 * 16, 18_048_737 // 16 * 16)
    copies = int(np.ceil(2e9 / sum(sizes)))
    bufs = [[torch.ones(b, dtype=torch.uint8, device=dev) for b in sizes] for _ in range(copies)]
    sinks = [[torch.empty(m.nvfp4moe_stream_blocks(b), dtype=torch.int32, device=dev)
              for b in sizes] for _ in range(copies)]

    def pair(i):
        for h in range(2):
            m.nvfp4moe_stream_read(bufs[i % copies][h], sink=sinks[i % copies][h])

    saved = args.steps
    args.steps = min(args.steps, 4000)
    ms, n = time_graph(pair, copies, args)
    args.steps = saved
    res["36MB+18MB"] = {"bytes": sum(sizes), "us": round(ms * 1e3, 3),
                        "GB/s": round(sum(sizes) / (ms * 1e-3) / 1e9, 1), "passes_timed": n,
                        "buffers_cycled": copies, "launches": 2}
    del bufs, sinks
    torch.cuda.empty_cache()
    gbs = res["4GiB"]["GB/s"]
    print(json.dumps({
        "metric": "HBM read ceiling GB/s (16-byte nontemporal loads, one pass)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": res["4GiB"]["passes_timed"],
        "warmup": args.warmup, "ms_per_step": round(res["4GiB"]["us"] / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic", "config": {"workload": "stream_read_ceiling",
                                         "timing": "hip graph replay, events"},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "sizes": res,
    }), flush=True)
    return 0


def timed_oracle(one, budget_s, threads):
    """Calls one(i) for i = 0, 1, ... with the oracle on `threads` threads
    until budget_s has passed: (calls, seconds, bytes summed from the calls'
    return values)."""
    import oracle
    saved = oracle.threads()
    oracle.set_threads(threads)
    try:
        done, nbytes, t0 = 0, 0, time.time()
        while True:
            b = one(done)
            if b is None:
                break
            nbytes += b
            done += 1
            if time.time() - t0 >= budget_s:
                break
        return done, time.time() - t0, nbytes
    finally:
        oracle.set_threads(saved)


def baseline_record(one, budget_s, rows_per_call, what):
    """The oracle single-threaded and on every usable host thread (at most
    16), each for about budget_s: the multi-threaded figure is the line's
    value, with the single-threaded one beside it."""
    import oracle
    T = oracle.default_threads()
    res = {}
    for t in (1, T):
        n, el, nb = timed_oracle(one, budget_s, t)
        res[t] = {"value": round(nb / el / 1e9, 5), "unit": "GB/s", "cores": t,
                  "rows_per_s": round(rows_per_call * n / el, 3), "seconds": round(el, 2),
                  "calls": n}
    top = res[T]
    return {"value": top["value"], "unit": "GB/s", "cores": T, "kind": "oracle",
            "rows_per_s": top["rows_per_s"], "seconds": top["seconds"],
            "sample": f"{top['calls']} {what} of the same workload on {T} threads "
                      f"(float64 oracle; output rows split over the threads)",
            "single_thread": res[1], **cpu_info()}


def cpu_baseline(layers_host, logit_sets, x_host, copies, n_sets, budget_s, shared, bias):
    """The oracle on the first steps of the same sequence (weight copy
    i % copies, logits/x set i % n_sets), single-threaded and threaded."""
    import oracle

    def one(i):  # the copies held on the host, in turn
        c, j = i % min(copies, len(layers_host)), i % n_sets
        lay = layers_host[c]
        L = logit_sets[j]
        ids, w, out = oracle.moe_decode(x_host[j], L.logits, lay.k, lay.gate_up, lay.down,
                                        bias=L.bias, shared_gate_up=lay.shared_gate_up,
                                        shared_down=lay.shared_down)
        return step_bytes(lay.M, lay.E, lay.k, lay.H, lay.I, len(np.unique(ids)), shared, bias)

    return baseline_record(one, budget_s, layers_host[0].M,
                           "decode steps (route + expert FFNs + combine)")


if __name__ == "__main__":
    sys.exit(main())
