"""Builds liboracle.so (the float64 CPU oracle) with g++. Test infrastructure."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off: every product and sum rounds on its own, as written
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-ffp-contract=off", "-fno-fast-math",
           "-pthread", os.path.join(HERE, "oracle.cpp"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
