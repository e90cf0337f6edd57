"""Build libmoe355.so in-tree with hipcc for gfx950.

    python -m expert_layer_amd.build        # compile every .hip, link the .so

Each source compiles to an object under ``_build/`` (in parallel), then the
objects are linked into ``expert_layer_amd/libmoe355.so``.  Packed fp32 vector
instructions are switched off for all device code.
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
OBJ = os.path.join(ROOT, "_build", "moe355")
LIB = os.path.join(PKG, "libmoe355.so")
ARCH = os.environ.get("MOE355_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with cf.ThreadPoolExecutor(jobs) as pool:
        objs = list(pool.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # a kernel whose host stub the compiler silently dropped links fine into a
    # shared library and only fails when it is loaded: refuse such a build
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.strip() for ln in nm.stdout.splitlines() if "moe355::" in ln]
    if nm.returncode != 0 or missing:
        raise RuntimeError("link left library symbols undefined:\n" + "\n".join(missing or [nm.stderr]))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
