"""Builds libnvfp4moe.so for gfx950 with hipcc (in-tree, no JIT cache)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4moe.so")
# the compiler's version lines, recorded beside the library at build time (a
# measurement reads them from here rather than running the compiler itself)
COMPILER_INFO = os.path.join(HERE, "libnvfp4moe.compiler.txt")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    v = subprocess.run([hipcc, "--version"], capture_output=True, text=True)
    with open(COMPILER_INFO, "w") as fh:
        fh.write("; ".join(l.strip() for l in v.stdout.splitlines() if "version" in l.lower()))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
