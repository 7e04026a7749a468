"""Build libtte.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m transformer_text_embedding_amd.build [--jobs N]
Every call recompiles; objects go to _build/ at the repository root and the
library to the package directory, where the Python binding loads it.
"""
from __future__ import annotations

import argparse
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
LIB = os.path.join(PKG, "libtte.so")
SOURCES = ["kernels_rows.hip", "kernels_gemm.hip", "kernels_attn.hip", "kernels_sim.hip", "tte.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions (v_pk_{add,mul,fma}_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# Per-source flags: matrix-core accumulators in ordinary VGPRs.  Left to
# itself the compiler parks accumulators in AGPRs whenever a kernel needs
# more than ~128 registers, and then moves them back and forth for every
# VALU touch: the attention's softmax, the int8 / 4-bit block-scale FMAs
# (which became ~50% more VALU instructions).  The bf16 GEMM kernels it
# leaves byte-identical.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCE_FLAGS = {"kernels_attn.hip": VGPR_FORM, "kernels_gemm.hip": VGPR_FORM}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    try:  # every kernel stub and export must resolve
        import ctypes
        ctypes.CDLL(tmp)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# CPU tier: the engine's host code (argument checks, workspace layout, pack
# validation, staging) with AddressSanitizer and UndefinedBehaviorSanitizer.
# Every -fsanitize= is a host-only flag: the device code is compiled as in
# the library, and nothing here runs on a GPU.
SANITIZE_DIR = os.path.join(BUILD, "host_sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libtte_host_sanitized.so")
SANITIZE_DRIVER = os.path.join(SANITIZE_DIR, "host_sanitizer_driver")
DRIVER_SRC = os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp")
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def host_clangxx() -> str:
    for c in ("/opt/rocm/llvm/bin/clang++", "/opt/rocm/lib/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("clang++ not found")


def build_host_sanitized(verbose: bool = False) -> str:
    """libtte_host_sanitized.so (tte.hip with the host sanitizers, linked
    with the regular kernel objects) and the driver that exercises its
    GPU-free paths; returns the driver's path."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    kernel_objs = []
    for src in SOURCES:
        if src == "tte.hip":
            continue
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        kernel_objs.append(obj if os.path.exists(obj) else _compile(src))
    obj = os.path.join(SANITIZE_DIR, "tte.o")
    cmd = [hipcc(), *HIPCC_FLAGS, *HOST_SANITIZE, "-c", os.path.join(CSRC, "tte.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on tte.hip (host sanitizers):\n{r.stdout}{r.stderr}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", SANITIZE_LIB, obj, *kernel_objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (host sanitizers):\n{r.stdout}{r.stderr}")
    # the driver is plain C++ (no HIP source), built by the host compiler
    cmd = [host_clangxx(), "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", INCLUDE, DRIVER_SRC, "-o", SANITIZE_DRIVER,
           "-L", SANITIZE_DIR, "-ltte_host_sanitized", f"-Wl,-rpath,{SANITIZE_DIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed:\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {SANITIZE_DRIVER}")
    return SANITIZE_DRIVER


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--host-sanitize", action="store_true",
                    help="also build the host-sanitizer library and driver (CPU tier)")
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    if a.host_sanitize:
        build_host_sanitized(verbose=True)
