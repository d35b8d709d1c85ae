"""Build the gfx950 HIP library libmoe_fp8.so in-tree.

    python -m mixture_experts_fp8_amd.build

Each .hip source is compiled by hipcc and each plain C++ source (.cpp: the host-side
validation and workspace arithmetic, which also builds without HIP) by the host compiler,
in parallel; the objects are linked into mixture_experts_fp8_amd/lib/libmoe_fp8.so.
Cross-compiles without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libmoe_fp8.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",   # no packed-fp32 VALU ops
    "-Wno-unused-result",
]


def _compile(src: str, obj: str) -> None:
    if src.endswith(".cpp"):
        cmd = [CXX, *CXXFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    errs = [ln for ln in r.stderr.splitlines() if "error" in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(OUT_DIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libmoe_fp8.so failed")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
