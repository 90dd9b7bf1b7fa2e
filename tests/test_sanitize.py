"""The oracle (oracle.c) and the C ABI's host code (argument checks, plans,
launch set-up in api.hip) under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: the oracle tests run against oracle.c built with gcc's sanitizers,
and the ABI tests against a copy of the library whose host code is built with
clang's.  Each suite runs in a child process with the matching runtime
preloaded; any report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _instrumented(lib):
    """The library calls into the sanitizer runtimes (it was built with them)."""
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    return "__asan_" in syms and "__ubsan_" in syms


def _run(env_extra, files):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:allocator_may_return_null=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *files], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_suite_under_gcc_asan_ubsan():
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    assert _instrumented(lib)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    files = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_"))
    out = _run({"DFS_ORACLE_LIB": lib, "LD_PRELOAD": asan}, files)
    assert " passed" in out


def test_abi_suite_with_host_code_under_clang_asan_ubsan():
    import glob

    from dictionary_factored_sparse_amd import build as hb
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    lib = hb.build_host_sanitized()
    assert _instrumented(lib)
    out = _run({"DFS_LIB_PATH": lib, "LD_PRELOAD": rt[-1]}, ["tests/test_abi.py"])
    assert " passed" in out
