"""Build libspecverify.so (the verify library) and libsvprobe.so (the
streaming-read ceiling probe that bench.py times beside it) for gfx950 with
hipcc, in-tree, next to this file."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "spec_verify.hip")
OUT = os.path.join(HERE, "libspecverify.so")
PROBE_SRC = os.path.join(HERE, "csrc", "read_probe.hip")
PROBE_OUT = os.path.join(HERE, "libsvprobe.so")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # Keep the backend from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc(src: str, out: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}) on {os.path.basename(src)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    """Compile both libraries (always); returns the verify library's path."""
    _hipcc(PROBE_SRC, PROBE_OUT, verbose)
    return _hipcc(SRC, OUT, verbose)


if __name__ == "__main__":
    print(build_library(verbose=True))
