"""Builds liboracle.so with the host C compiler (test infrastructure only).

Flags follow the oracle's contract: no fast-math and no contraction of a
multiply and an add into an FMA, so every float operation rounds as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
# the same source evaluated in two other valid ways (used only to measure a
# workload's sensitivity to the rounding of its sums): every dot product summed
# over i descending, and every sum accumulated in double and rounded once
LIB_DESC = os.path.join(HERE, "liboracle_desc.so")
LIB_F64 = os.path.join(HERE, "liboracle_f64.so")
VARIANTS = {"": (LIB, []), "desc": (LIB_DESC, ["-DORC_DOT_DESCENDING"]), "f64": (LIB_F64, ["-DORC_SUM_F64"])}
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11", "-Wall", "-Wno-unused-function"]


def _build_one(out: str, extra, verbose: bool) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, "-shared", "-fPIC", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    for name, (out, extra) in VARIANTS.items():
        if name:
            _build_one(out, extra, verbose)
    return _build_one(LIB, [], verbose)


if __name__ == "__main__":
    print(build(verbose=True))
