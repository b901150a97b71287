"""Compile the HIP sources under csrc/ into libfa.so (gfx950) in this directory.

Usage: python -m exact_io_aware_10_amd.build   (or build() from Python)
Object files go to _build/ at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_atomic.hip", "fa_fp8.hip"]
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if src.endswith(".hip"):
        _check_asm(src)
    return obj


def _check_asm(src: str) -> None:
    """Verify the inline-assembly MFMAs of one source in its generated code."""
    from . import asm_check

    asm = os.path.join(BUILD, os.path.basename(src) + ".s")
    cmd = [HIPCC, *COMMON, "-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src),
           "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    with open(asm) as f:
        problems = asm_check.check(f.read())
    if problems:
        raise RuntimeError(f"{src}: inline-assembly hazards:\n" + "\n".join(problems))


MICRO_SRC = os.path.join(ROOT, "micro", "micro.hip")
MICRO_BIN = os.path.join(ROOT, "micro", "micro")


def build_micro(verbose: bool = False) -> str:
    """The microbenchmark program (micro/micro.hip) behind the rates the kernels'
    design relies on; a standalone executable, not part of the library."""
    cmd = [HIPCC, *COMMON, "-munsafe-fp-atomics", MICRO_SRC, "-o", MICRO_BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for micro.hip:\n{r.stderr}")
    if verbose:
        print(f"built {MICRO_BIN}")
    return MICRO_BIN


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    build_micro(verbose=True)
    sys.exit(0)
