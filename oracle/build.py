"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

Plain C11, -O2, no fast-math and no FMA contraction, so every double operation is the
one written in oracle.c.  OpenMP only spreads independent rows/heads over threads.

`python oracle/build.py --sanitize` builds oracle/liboracle_san.so instead, with AddressSanitizer
and UndefinedBehaviorSanitizer (host code, gcc); the CPU tests run against it with

    LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    VOX_ORACLE_LIB=oracle/liboracle_san.so python -m pytest tests -m "not gpu"
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if sanitize:
        cmd[2:2] = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
