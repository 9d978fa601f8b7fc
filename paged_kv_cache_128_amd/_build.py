"""Build libpkv.so (HIP kernels for gfx950 + the host block manager) in-tree.

    python -m paged_kv_cache_128_amd._build

Every call compiles from source.  The library lands in
``paged_kv_cache_128_amd/_lib/libpkv.so`` next to the Python binding that
loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libpkv.so")
OBJDIR = os.path.join(ROOT, "_build", "pkv")

ARCH = "gfx950"
SOURCES = ["pkv_kernels.hip", "pkv_blocks.hip", "pkv_fp8.hip", "pkv_prefill.hip", "manager.cpp"]
# Packed fp32 ops (v_pk_*_f32) are switched off for every device pass.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
          "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpkv)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs = []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"] if src.endswith(".hipx") else []
        out = _run([cc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
