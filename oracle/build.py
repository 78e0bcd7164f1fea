"""Build the CPU oracle shared library (oracle/liboracle.so) with gcc.

Test infrastructure only: the library built here is loaded by the test suite,
the package smoke check and the CPU-baseline leg of the benchmark, never by the
GPU library.  Flags keep the arithmetic plain IEEE fp64: no fast-math and no
contraction of a*b+c into fused multiply-adds.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
