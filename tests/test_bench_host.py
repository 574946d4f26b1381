"""Host-side checks of bench.py (no GPU): its byte accounting against the
shapes' own arithmetic, and its refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_expert_bytes_of_the_block_shape():
    # gate_up [1024][2048] and down [2048][512] in NVFP4: a 4-bit code per
    # weight, an E4M3 byte per 16 weights, one FP32 tensor scale per matrix
    gu = 1024 * 2048 // 2 + 1024 * 2048 // 16 + 4
    dn = 2048 * 512 // 2 + 2048 * 512 // 16 + 4
    assert (gu, dn) == (1_179_652, 589_828)
    assert bench.expert_bytes(2048, 512) == gu + dn == 1_769_480
    # 256 experts per block, 40 blocks: about 18.1 GB of packed experts
    assert abs(40 * 256 * bench.expert_bytes(2048, 512) / 1e9 - 18.12) < 0.01


def test_step_bytes_terms():
    e = bench.expert_bytes(2048, 512)
    # M=4, 30 experts touched, no shared expert, no bias, grouping arrays read
    b = bench.step_bytes(4, 256, 8, 2048, 512, 30, False, False)
    acts = 4 * 2048 * 2 * 2 + 4 * 256 * 4 + 4 * 8 * 8 * 2
    grouping = (256 + 257 + 257) * 4 + 4 * 8 * 4 * 2
    assert b == 30 * e + acts + grouping
    # routing folded in: no grouping arrays; a shared expert adds one expert's bytes
    assert bench.step_bytes(4, 256, 8, 2048, 512, 30, False, False, grouped=False) == \
        30 * e + acts
    assert bench.step_bytes(4, 256, 8, 2048, 512, 30, True, True, grouped=False) == \
        31 * e + acts + 256 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
