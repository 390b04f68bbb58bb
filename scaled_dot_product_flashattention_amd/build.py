"""Build ``libattn.so`` (the HIP kernels and their C ABI) for gfx950, in-tree.

Each source is compiled to an object under ``_build/`` in parallel, then the
objects are linked into ``scaled_dot_product_flashattention_amd/libattn.so``.
All device code is built without packed-fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["attn_api.cpp", "fwd_prefill.hip", "fwd_prefill16.hip", "fwd_splitk.hip", "naive.hip",
           "qkv_proj.hip", "softmax_rows.hip", "noalloc.hip"]
ARCH = os.environ.get("ATTN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set HIPCC or install ROCm")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # inputs are finite by contract; lets fmaxf skip NaN canonicalisation
        # (infinities keep their full semantics)
        "-fno-honor-nans",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def library_path() -> str:
    return os.path.join(PKG, "libattn.so")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    out = library_path()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libattn.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(out + ".tmp", out)
    if verbose:
        print(out)
    return out


if __name__ == "__main__":
    build(verbose=True)
