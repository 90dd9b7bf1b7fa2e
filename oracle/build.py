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


SAN_LIB = os.path.join(HERE, "liboracle_san.so")
# AddressSanitizer and UndefinedBehaviorSanitizer (CPU only); a UB report aborts
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build liboracle.so, or with sanitize=True liboracle_san.so (load it
    with DFS_ORACLE_LIB pointing at it and gcc's libasan preloaded)."""
    out = SAN_LIB if sanitize else LIB
    cmd = ["gcc", "-std=c11", "-O1" if sanitize else "-O2", "-fopenmp", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", *(SAN_FLAGS if sanitize else []),
           "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
