"""Build libqmv.so (the gfx950 HIP kernels behind include/qmv.h) in-tree.

hipcc cross-compiles for gfx950 without a GPU. Every source is compiled with
packed-FP32 instruction selection turned off; the library links only the HIP
runtime (the same libamdhip64.so.7 soname torch loads, so one runtime serves
both).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libqmv.so")
BUILD = os.path.join(HERE, "_build")

HIP_SOURCES = ["qmv_dense.hip", "qmv_q8act.hip", "moe.hip", "qmm.hip", "gate.hip", "roofline.hip"]
CPP_SOURCES = ["misc.cpp"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]
HIP_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc"]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    flags = COMMON + (HIP_FLAGS if src.endswith(".hip") else ["-x", "c++"])
    cmd = [_hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "unknown target feature" not in l and "packed-fp32" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, HIP_SOURCES + CPP_SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
