"""Build the HIP shared library ``libnvfp4q.so`` in-tree for gfx950.

Usage: ``python -m rmsnorm_nvfp4_block_amd.build`` (or ``build()`` from Python).
Each ``.hip`` translation unit is compiled in parallel into ``_build/`` and
linked into ``rmsnorm_nvfp4_block_amd/libnvfp4q.so``; the measurement probes
(``csrc/ceilings.hip``, used only by ``bench.py --ceilings``) go into
``libnvfp4q_ceilings.so`` beside it. Flags: -O3, gfx950 only,
no FMA contraction (the quantizer's products must round on their own), NaN
handling off (inputs are finite by contract; it removes NaN canonicalization
around max), and the packed-FP32 feature disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnvfp4q.so")
CEIL_LIB = os.path.join(HERE, "libnvfp4q_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]
SOURCES = [
    "api.hip", "kernels_rows.hip", "kernels_rms_coop.hip",
    "kernels_rms_stream.hip",
    "kernels_2d.hip", "kernels_grouped.hip", "kernels_qk.hip",
]
ARCH = "gfx950"

COMMON = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEIL_LIB)
    if verbose:
        print("built", LIB, "and", CEIL_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
