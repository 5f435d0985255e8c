"""Builds the in-tree HIP library ``libw4.so`` for gfx950 with hipcc.

Each source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel), then linked into ``bit_weight_quantized_amd/libw4.so``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(PKG_DIR), "_build")
LIB_PATH = os.path.join(PKG_DIR, "libw4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # Packed-fp32 VALU forms stay disabled; ordinary float code is used.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON_FLAGS, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip() and os.environ.get("W4_BUILD_VERBOSE"):
        sys.stderr.write(r.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libw4.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
