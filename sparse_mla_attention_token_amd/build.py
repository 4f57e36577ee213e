"""Build the gfx950 shared library (libsmla.so) in-tree with hipcc.

Each source is compiled to its own object (in parallel), then the objects are
linked into one shared library.  Per-source flags: the kernels whose P.V
accumulators live in AGPRs while their score accumulators are written as VGPR
instructions are compiled without the VGPR-form MFMA selection the others use.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libsmla.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # never let the compiler form packed f32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]

# select the VGPR form of every MFMA and let the allocator move only the
# long-lived P.V accumulators to AGPRs (the all-AGPR form overflows them)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]

# sources built without VGPR_FORM: their score MFMAs are VGPR instructions
# already and the P.V accumulators take all 256 AGPRs
NO_VGPR_FORM = {"smla_f16w.hip"}

LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC", "-fvisibility=hidden"]


def sources():
    return sorted(CSRC.glob("*.hip"))


def flags_for(src: Path):
    extra = [] if src.name in NO_VGPR_FORM else VGPR_FORM
    return [*COMMON_FLAGS, *extra, "-I", str(PKG.parent / "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[-3:])}")


PROBE_SRC = PKG / "probe" / "smla_probe.hip"
PROBE_LIB = PKG / "libsmla_probe.so"


def build_probe(verbose: bool = False) -> Path:
    """The measurement probes (MFMA peak, row-gather rate): libsmla_probe.so."""
    tmp = PROBE_LIB.with_suffix(".so.tmp")
    _run([HIPCC, *COMMON_FLAGS, "-shared", "-I", str(PKG.parent / "include"), str(PROBE_SRC), "-o", str(tmp)],
         verbose)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> Path:
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with tempfile.TemporaryDirectory(prefix="smla_build_") as tmpdir:
        objs = [Path(tmpdir) / (s.stem + ".o") for s in srcs]
        cmds = [[HIPCC, *flags_for(s), "-c", str(s), "-o", str(o)] for s, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB.with_suffix(".so.tmp")
        _run([HIPCC, *LINK_FLAGS, *map(str, objs), "-o", str(tmp)], verbose)
        os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
