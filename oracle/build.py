"""Builds liboracle.so with the host C compiler (test infrastructure only).

Flags follow the oracle's contract: no fast-math and no contraction of a
multiply and an add into an FMA, so every float operation rounds as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11", "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
