"""Build libtpcolpar.so (HIP for gfx950) in-tree, next to this file.

    python -m megatron_tensor_transformer_colpar_amd.build

Each source compiles to an object under ``_build/`` (in parallel), then hipcc
links the shared library.  Every HIP source is built with packed-fp32 ops
disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtpcolpar.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ROCM_INCLUDE = "/opt/rocm/include"
ARCH = "gfx950"

SOURCES = ["gemm_bf16.hip", "gemv_bf16.hip", "gemm_f32.hip", "attn_bf16.hip", "reduce.hip", "scratch.hip", "plan.cpp", "abi.cpp"]
COMMON = ["-O3", "-std=c++20", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
HIP_ONLY = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OUT_DIR, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_ONLY, *COMMON, "-c", path, "-o", obj]
    else:  # host-only C++ (the C ABI): no device code, plain g++
        cmd = [CXX, *COMMON, "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def _check_no_missing_stubs(lib: str) -> None:
    """Fail if the host pass dropped a kernel's launch stub (the library would
    link, then refuse to load)."""
    r = subprocess.run(["nm", "-u", "-C", lib], capture_output=True, text=True)
    missing = [l.strip() for l in r.stdout.splitlines() if "tpk::" in l]
    if missing:
        raise RuntimeError("libtpcolpar.so references undefined library symbols:\n" + "\n".join(missing))


def build(verbose: bool = False) -> str:
    """Compile every source and link libtpcolpar.so; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    try:
        _check_no_missing_stubs(tmp)
    except RuntimeError:
        os.remove(tmp)
        raise
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
