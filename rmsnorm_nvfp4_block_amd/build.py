"""Build the HIP shared library ``libnvfp4q.so`` in-tree for gfx950.

Usage: ``python -m rmsnorm_nvfp4_block_amd.build`` (or ``build()`` from Python);
``python -m rmsnorm_nvfp4_block_amd.build --sanitize`` builds the library with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (into
``_build/sanitize/``; device code is built as usual) and runs the CPU tests of
the C ABI (``tests/test_abi_cpu.py``: argument validation, nothing launched)
against it with the sanitizer runtime preloaded. It needs no GPU.
Each ``.hip`` translation unit is compiled in parallel into ``_build/`` and
linked into ``rmsnorm_nvfp4_block_amd/libnvfp4q.so``, which carries the sha256 of
the sources it was built from (``source_digest()``: every file of ``csrc/`` and
``include/``; ``nvfp4q_source_sha256()`` in the C ABI), so a prebuilt library
can be checked against the tree; the measurement probes
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


def source_digest() -> str:
    """sha256 over the library's sources: every file of csrc/ and include/, by name and content."""
    import hashlib

    h = hashlib.sha256()
    inc = os.path.join(ROOT, "include")
    for d in (CSRC, inc):
        for f in sorted(os.listdir(d)):
            path = os.path.join(d, f)
            if os.path.isfile(path) and f.endswith((".hip", ".hpp", ".h")):
                h.update(f.encode() + b"\0")
                with open(path, "rb") as fh:
                    h.update(fh.read())
                h.update(b"\0")
    return h.hexdigest()


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, f'-DNVFP4Q_SOURCE_SHA256="{digest}"', "-c", os.path.join(CSRC, src), "-o", obj]
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
    digest = source_digest()
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda f: _compile(f, digest), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CEIL_LIB)
    if verbose:
        print("built", LIB, "and", CEIL_LIB)
    return LIB


# Host-only sanitizers: every -fsanitize= sits behind -Xarch_host, so no GPU
# code is built with them.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _asan_runtime() -> str:
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "/opt/rocm/llvm/bin/clang"
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    for sub in ("lib/linux", "lib/x86_64-unknown-linux-gnu"):
        p = os.path.join(res, sub, "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError(f"no AddressSanitizer runtime under {res}")


def sanitize_check() -> int:
    """Host-sanitized build of the library, then the CPU ABI tests against it. Returns pytest's status."""
    out = os.path.join(BUILD, "sanitize")
    os.makedirs(out, exist_ok=True)
    digest = source_digest()

    def comp(src: str) -> str:
        obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *COMMON, *SANITIZE, f'-DNVFP4Q_SOURCE_SHA256="{digest}"', "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(comp, SOURCES))
    lib = os.path.join(out, "libnvfp4q.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    rt = _asan_runtime()
    runner = (
        "import sys; sys.path.insert(0, %r); import rmsnorm_nvfp4_block_amd as q; q.lib_path = %r; "
        "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))"
        % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    env = dict(os.environ, LD_PRELOAD=rt, LD_LIBRARY_PATH=os.path.dirname(rt),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    print("sanitized library:", lib, "\nruntime:", rt, flush=True)
    return subprocess.run([sys.executable, "-c", runner], env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        sys.exit(sanitize_check())
    build(verbose=True)
    sys.exit(0)
