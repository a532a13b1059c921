"""Builds libdspark.so (HIP kernels for gfx950 + the C ABI) in this directory.

Usage: python -m semi_ar_drafter_amd.build_lib  (or __graft_entry__.build()).
Always recompiles.  Object files go to _build/ beside the sources.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
# Packed fp32 instructions stay disabled in all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    ("api.cpp", False),
    ("markov_draft.hip", True),
    ("schedule_verify.hip", True),
    ("parallel_draft.hip", True),
    ("sts_fit.hip", True),
]
# Per-source flags.  The draft kernel's inputs are finite by contract, so its
# maxima need not quiet signalling NaNs (no canonicalising instruction before
# every v_max_f32).
EXTRA = {"markov_draft.hip": ["-fno-honor-nans"]}


def _compile(src: str, device: bool) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + (DEVICE + ["-x", "hip"] if device else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]) + \
          ["-I", os.path.join(HERE, "..", "include"), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(*s), SOURCES))
    lib = os.path.join(HERE, "libdspark.so")
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
