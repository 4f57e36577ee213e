"""Build the gfx950 shared library (libsmla.so) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libsmla.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # never let the compiler form packed f32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # select the VGPR form of every MFMA and let the allocator move only the
    # long-lived P.V accumulators to AGPRs (the all-AGPR form overflows them)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]


def sources():
    return sorted(CSRC.glob("*.hip"))


def build(verbose: bool = False) -> Path:
    srcs = [str(s) for s in sources()]
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, *HIP_FLAGS, "-I", str(PKG.parent / "include"), *srcs, "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
