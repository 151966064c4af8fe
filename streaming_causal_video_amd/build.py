"""Compile the HIP kernels and the C-ABI host library into ``liblahip.so`` (gfx950).

Usage: ``python -m streaming_causal_video_amd.build`` (or ``build()``).  Each
source is compiled to an object with hipcc in parallel, then linked into a
shared library next to this file.  The build always runs (no staleness check),
so callers that changed a source get a fresh library.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "liblahip.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["la_api.cpp", "rope.hip", "stream_ops.hip", "attn_bf16.hip", "attn_fp8.hip",
           "attn_f32.hip", "noalloc.hip"]

# Per-source extra flags.  The attention kernels never see NaN inputs, so they are
# built without NaN-quieting semantics: fmaxf then maps to bare v_max/v_max3
# instead of canonicalising every operand first.
EXTRA = {"attn_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
         "attn_fp8.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}

# hipcc flags.  Packed-fp32 instruction selection is switched off for device code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *CFLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link liblahip.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
