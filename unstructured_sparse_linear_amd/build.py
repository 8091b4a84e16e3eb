"""Build libspops.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into libspops.so next to this file.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "spops")
LIB = os.path.join(HERE, "libspops.so")
CEILINGS_LIB = os.path.join(HERE, "libspops_ceilings.so")
ARCH = os.environ.get("SPOPS_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 VALU forms stay off: ordinary fp32 code is emitted instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    build_ceilings(verbose)
    return LIB


def build_ceilings(verbose: bool = False) -> str:
    """The benchmark's measurement kernels (gather rates), a library of their
    own that libspops does not link."""
    src = os.path.join(HERE, "ceilings", "ceilings.hip")
    obj = _compile(src)
    tmp = CEILINGS_LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, CEILINGS_LIB)
    if verbose:
        print(f"built {CEILINGS_LIB}", file=sys.stderr)
    return CEILINGS_LIB


if __name__ == "__main__":
    build(verbose=True)
