"""Build libvpk.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m varlen_paged_kv_amd.build        # or: python varlen_paged_kv_amd/build.py

Every source is compiled with hipcc for --offload-arch=gfx950; packed fp32
instructions are disabled in device code (-packed-fp32-ops).  The library is
written to varlen_paged_kv_amd/lib/libvpk.so; the benchmark's read-bandwidth
helper to varlen_paged_kv_amd/lib/libvpk_measure.so.
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
OUT_DIR = os.path.join(HERE, "lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(OUT_DIR, "libvpk.so")
# a separate helper library for the benchmark's read-bandwidth reference (not
# part of the attention path; only bench.py loads it)
MEASURE_LIB = os.path.join(OUT_DIR, "libvpk_measure.so")
MEASURE_SOURCES = ["measure/read_bw.hip"]

SOURCES = [
    "kernels/attn_fwd.hip",
    "kernels/append.hip",
    "kernels/merge.hip",
    "kernels/rope.hip",
    "kernels/scratch.hip",
    "host/plan.cpp",
    "host/abi.cpp",
]

ARCH = os.environ.get("VPK_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvpk)")


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src.replace("/", "_") + ".o")
    cmd = [hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + MEASURE_SOURCES
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], MEASURE_LIB)
    if verbose:
        print("built", LIB, "and", MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
