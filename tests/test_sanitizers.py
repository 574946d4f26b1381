"""CPU builds of the oracle and of the C ABI's host-side validation with
AddressSanitizer and UndefinedBehaviorSanitizer, run on small inputs (no
GPU): an out-of-bounds access, a leak (oracle) or an undefined operation
(signed overflow in the size arithmetic, a bad shift) fails the run.
The HIP library's device code is built as usual; only its host code is
instrumented, and every ABI call made is one its validation rejects before
any launch."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", *SAN, "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-pthread", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "oracle", "oracle.cpp"),
                    os.path.join(HERE, "oracle_main.cpp"), "-o", exe], check=True)
    assert "ok" in _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})


HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    host_san = []
    for flag in SAN:  # host code only: the device code is not instrumented
        host_san += ["-Xarch_host", flag]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "nvfp4_moe_skinny_amd", "csrc"),
                    os.path.join(ROOT, "nvfp4_moe_skinny_amd", "csrc", "api.hip"),
                    os.path.join(HERE, "abi_main.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    # the HIP runtime's own allocations are not the library's: no leak check
    assert "ok" in _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
