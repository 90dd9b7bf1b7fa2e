"""Build the CPU oracle (``oracle/liboracle.so``) with gcc.

Test infrastructure: the library built here is loaded only by the tests,
the smoke check and the benchmark's CPU-baseline leg.

No -ffast-math and -ffp-contract=off: the NVFP4 encoder's fp32 steps must be
individually rounded operations, and x86-64 float arithmetic (SSE) gives
exactly that.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
