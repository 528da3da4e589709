"""Build the in-tree HIP library ``libkvq.so`` for gfx950.

Usage: ``python -m decode_attention_quantized_amd.build`` (or ``build()``).
Every call recompiles; objects go to ``_build/`` at the repository root.
The packer is plain C++ (compiled without FMA contraction so every rounding
step is the written one); kernels and host entry points go through hipcc.
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
LIB = os.path.join(PKG, "libkvq.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}"]
# every HIP translation unit: no packed fp32 instructions
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    ("kvq_pack.cpp", ["-x", "c++", "-ffp-contract=off", "-fno-fast-math"]),
    ("kvq_api.cpp", HIP_FLAGS),
    # the kernels never produce or test NaN; without NaN semantics fmaxf
    # needs no input quieting and folds into DPP reductions
    ("kvq_gqa.hip", HIP_FLAGS + ["-ffp-contract=fast", "-fno-honor-nans"]),
    ("kvq_mla.hip", HIP_FLAGS + ["-ffp-contract=fast", "-fno-honor-nans"]),
    # the device packer rounds exactly as the host packer: no contraction
    ("kvq_append.hip", HIP_FLAGS + ["-ffp-contract=off", "-fno-fast-math"]),
    # streaming-read reference used by the measurements
    ("kvq_probe.hip", HIP_FLAGS),
]


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".cpp") and "-x" in extra:
        cmd = [HIPCC] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [HIPCC] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libkvq.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(*s), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
