"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

Plain C11, -O2, no fast-math and no FMA contraction, so every double operation is the
one written in oracle.c.  OpenMP only spreads independent rows/heads over threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
