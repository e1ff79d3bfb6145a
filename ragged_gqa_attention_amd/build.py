"""Builds the gfx950 shared library ``libragged_gqa_attn.so`` in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked.  All
HIP code is built with packed-FP32 instructions disabled (the compiler would
otherwise form v_pk_* FP32 ops on its own).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libragged_gqa_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = (["api.cpp", "plan.hip", "noalloc.hip"] +
           [f"{k}_d{d}.hip" for k in ("fwd", "dkdv", "dq") for d in (64, 128, 160)])
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = _flags() + list(extra_flags)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + flags + ["-c"] + lang + [os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = [ln for ln in (res.stderr or "").splitlines()
                 if "packed-fp32-ops' is not a recognized feature" not in ln]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
