"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain C, -O2, no fused multiply-add contraction, no fast-math, OpenMP over
independent rows.  Run as ``python oracle/build.py`` or via
``__graft_entry__.build()``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
