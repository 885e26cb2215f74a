"""Compile the HIP library (libsla.so) for gfx950, in-tree.

Each csrc/*.hip file is compiled to an object under _build/ (in parallel) and
linked into differentiable_sparse_linear_csr_amd/libsla.so. Device code is
built without packed-fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsla.so")
ARCH = "gfx950"

SOURCES = ["util.hip", "assembly.hip", "spmv.hip", "pcg.hip", "bicgstab.hip", "resident.hip",
           "reorder.hip",
           "seg.hip", "noalloc.hip", "api.hip"]
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsla.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


C_EXAMPLE = os.path.join(ROOT, "tests", "c", "abi_solve.c")


def build_c_example(verbose: bool = False) -> str:
    """The plain-C program the ABI test runs (links libsla.so and the HIP
    runtime; no C++ and no PyTorch)."""
    out = os.path.splitext(C_EXAMPLE)[0]
    clang = "/opt/rocm/llvm/bin/clang"
    cmd = [clang if os.path.exists(clang) else "clang", "-x", "c", "-std=c99", "-O2", "-Wall",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{INCLUDE}", C_EXAMPLE, "-o", out,
           f"-L{PKG}", "-lsla", "-L/opt/rocm/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../differentiable_sparse_linear_csr_amd",
           "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building {C_EXAMPLE} failed:\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libsla.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    if os.path.exists(C_EXAMPLE):
        build_c_example(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
