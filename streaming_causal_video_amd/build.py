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


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (it also carries UBSan)."""
    import glob
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib",
                                          "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("clang's shared ASan runtime was not found")
    return found[-1]


def build_host_sanitized(out_dir: str) -> str:
    """A CPU-side checking build: the host library code (la_api.cpp: argument checks,
    ring and sink state, the step and chain drivers) compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer for the host only, linked with the ordinary kernel
    objects of the last build().  Returns the library path; load it into a process
    that has asan_runtime() preloaded.  Not for GPU runs."""
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES[1:]]
    if not all(os.path.exists(o) for o in objs):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = os.path.join(out_dir, "la_api_san.o")
    cmd = [hipcc(), *[f for f in CFLAGS if f != "-O3"], "-O1", "-g", *san, "-x", "hip", "-c",
           os.path.join(CSRC, SOURCES[0]), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{res.stderr}")
    rocm = os.path.dirname(os.path.dirname(hipcc()))
    lib = os.path.join(out_dir, "liblahip_san.so")
    cmd = [os.path.join(rocm, "llvm", "bin", "clang++"), "-shared", "-fsanitize=address,undefined",
           "-shared-libsan", api_obj, *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stderr}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
