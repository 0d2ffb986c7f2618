"""Builds libsynth.so, the seeded input generator, with the host C compiler."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "synth.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
