"""Build libqmx.so in-tree with hipcc for gfx950.

    python -m matmul_affine_qmv_amd.build [-j JOBS]

Each source is compiled to an object under ``_build/`` (in parallel), then
linked into ``matmul_affine_qmv_amd/libqmx.so``; the calibration kernels
(``csrc/calib.hip``) go into ``libqmx_calib.so`` beside it.  Every call
compiles again; nothing is cached.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmx.so")
CALIB_LIB = os.path.join(PKG, "libqmx_calib.so")

SOURCES = ["qmv.hip", "qmm_b4.hip", "qmm_b8.hip", "qmm_b2.hip", "qmm_b3.hip", "qmm_b6.hip", "qmm_b5.hip",
           "qmm_b1.hip", "blocks.hip", "q8_i8.hip", "qmm.hip", "qmx_api.cpp", "noalloc.hip"]
CALIB_SOURCES = ["calib.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are kept out of every device build.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)


if __name__ == "__main__":
    main()
