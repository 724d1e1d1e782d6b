"""Compile the fp64 CPU oracle (test infrastructure) into oracle/liborc.so.

Plain C11 + libm + OpenMP with gcc; no fast-math, so sums keep the order the
source writes.  Used by the test-suite, the smoke check and the benchmark's
CPU-baseline leg only.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liborc.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "orc.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
