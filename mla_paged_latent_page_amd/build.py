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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources(src_dir=SRC_DIR):
    return sorted(glob.glob(os.path.join(src_dir, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_library(out, srcs, include_dir, verbose=False, jobs=8):
    """Compile each source to an object, in parallel, then link the objects
    into the shared library `out`."""
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = out + ".objs"
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(i):
        _run([HIPCC, *FLAGS, "-I", include_dir, "-c", "-o", objs[i], srcs[i]], verbose)

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(compile_one, range(len(srcs))))
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into the shared library, and the measurement
    kernels into their own (always recompiles)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = os.path.join(ROOT, "include")
    build_library(LIB_PATH, sources(), inc, verbose)
    build_library(PEAKS_PATH, sorted(glob.glob(os.path.join(SRC_DIR, "peaks", "*.hip"))), inc, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
