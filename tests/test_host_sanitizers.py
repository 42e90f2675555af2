"""The library's host half (argument checks, the plan of parts per row, the
workspace layout, the entry points' early returns) built with
AddressSanitizer and UndefinedBehaviorSanitizer, its device code as in the
product build, and the ABI tests run against that build in a child process
with the sanitizer runtime preloaded: any report fails the child.  CPU only:
no call in those tests reaches a GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "speculative_sampling_verification_verify_amd", "csrc", "spec_verify.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _runtime() is None, reason="hipcc or the ASan runtime is missing")
def test_abi_tests_under_host_sanitizers(tmp_path):
    lib = str(tmp_path / "libspecverify_hostsan.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libsan",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-o", lib, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-4000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
    env = dict(os.environ, SV_LIBRARY=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
