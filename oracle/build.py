"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc: the
definitions (mxfp8_oracle.c) and the error budget of a hardware accumulation (accum_bound.c).

Plain C11 + OpenMP, -O2, no fast-math: the oracle's floating point must follow
IEEE fp64 exactly as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "mxfp8_oracle.c"), os.path.join(HERE, "accum_bound.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", *SRCS, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
