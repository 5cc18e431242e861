"""Build libpa.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_118_amd.build

Every HIP source gets ``-Xclang -target-feature -Xclang -packed-fp32-ops``
(packed fp32 instructions are kept out of the generated code).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Per-source code generation options.  The chunked-prefill kernel keeps its
# MFMA accumulators in ordinary VGPRs: with accumulation registers the compiler
# copied all of them to VGPRs on every key group.
EXTRA_FLAGS = {"prefill_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj: str) -> None:
    is_hip = src.endswith(".hip")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    if is_hip:
        cmd[1:1] = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-ffp-contract=fast", "-munsafe-fp-atomics"]
        cmd[1:1] = EXTRA_FLAGS.get(os.path.basename(src), [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")


def build_library(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host allocator alone (alloc.cpp with sha256.h), built with g++ under
# AddressSanitizer and UndefinedBehaviorSanitizer, for running the CPU test
# suites against it: PA_ALLOC_LIB=<this .so> routes the binding's pa_alloc_*
# and pa_prefix_block_hash there; the process needs gcc's libasan preloaded
# (LD_PRELOAD=$(gcc -print-file-name=libasan.so)).  CPU only.
SAN_LIB = os.path.join(BUILD, "san", "libpa_alloc_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
             "-g", "-O1"]


def build_sanitized_alloc() -> str:
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    tmp = SAN_LIB + f".tmp{os.getpid()}"
    cmd = ["g++", "-std=c++17", "-shared", "-fPIC", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "alloc.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build_sanitized_alloc())
    else:
        print(build_library())
