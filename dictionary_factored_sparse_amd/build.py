"""Build ``libdictfs.so`` (the HIP library behind include/dictfs.h) for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` in parallel,
then linked into ``dictionary_factored_sparse_amd/libdictfs.so``.  hipcc
cross-compiles for gfx950 without a GPU.

Flags: -O3, no fast-math, fp32 denormals kept, correctly rounded fp32
division (hipcc's default), packed-fp32 instructions disabled.  The NVFP4
encoder is compiled with -ffp-contract=off so that each step of its recipe
is one rounded operation.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdictfs.so")
ARCH = os.environ.get("DFS_OFFLOAD_ARCH", "gfx950")

COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PER_FILE = {"nvfp4.hip": ["-ffp-contract=off"], "quant8.hip": ["-ffp-contract=off"]}


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "san", "libdictfs.so")
# host code only: every -fsanitize= applies to the host pass (-Xarch_host);
# device code is unchanged
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def build_host_sanitized(verbose: bool = False) -> str:
    """A copy of the library whose host code (the C ABI's argument checks,
    plans and launches, all in api.hip) is built with AddressSanitizer and
    UndefinedBehaviorSanitizer, for CPU tests (load it with DFS_LIB_PATH and
    clang's ASan runtime preloaded).  Reuses the other objects of build()."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    others = [os.path.join(BUILD, os.path.basename(f) + ".o")
              for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
              if os.path.basename(f) != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        build(verbose)
    obj = os.path.join(os.path.dirname(SAN_LIB), "api.hip.o")
    cmd = [_hipcc(), *COMMON, *SAN_HOST, "-c", os.path.join(CSRC, "api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on api.hip (sanitized):\n{r.stderr}")
    r = subprocess.run([_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", SAN_LIB + ".tmp", obj,
                        *others], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build_host_sanitized(verbose=True) if "--sanitize" in sys.argv
          else build(verbose="-v" in sys.argv))
