"""Build the gfx950 HIP library ``_build/libmla_paged.so`` in-tree with hipcc,
and the measurement kernels bench.py reports ceilings with
(``_build/libmla_peaks.so``, from ``csrc/peaks/``; not part of the path)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC_DIR = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libmla_paged.so")
PEAKS_PATH = os.path.join(BUILD_DIR, "libmla_peaks.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(SRC_DIR, "*.hip")))


def _hipcc(out, srcs, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into the shared library, and the measurement
    kernels into their own (always recompiles)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    _hipcc(LIB_PATH, sources(), verbose)
    _hipcc(PEAKS_PATH, sorted(glob.glob(os.path.join(SRC_DIR, "peaks", "*.hip"))), verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
