"""Build the gfx950 library ``libnormgemm.so`` in-tree with hipcc.

Usage: ``python norm_gemm_amd/build.py`` (also called by the repository's
build entry point). Every HIP source is compiled for gfx950 only; the C
validation layer is compiled as plain host C. Objects go to
``norm_gemm_amd/_build/``; the library is written next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnormgemm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU forms are left to no one: the target feature is disabled
# for every device compile.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-mcode-object-version=5", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{INCLUDE}", f"-I{CSRC}"]
C_FLAGS = ["-O2", "-std=c11", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}"]

SOURCES = ["api.cpp", "prefill.hip", "prefill_lds.hip", "decode.hip", "decode_lds.hip", "decode_wide.hip",
           "gated.hip", "prefill_wide.hip", "fold.hip", "postnorm.hip"]
C_SOURCES = ["validate.c", "route.c"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".c"):
        cmd = ["gcc", *C_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *HIP_FLAGS, "-x", "hip", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + C_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
