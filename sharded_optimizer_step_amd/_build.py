"""Build the library of the per-rank ZeRO shard step in-tree: the gfx950 HIP
kernels and the C ABI with hipcc (it cross-compiles without a GPU), the host
optimizer of the CPU-offloaded step with g++."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "zero_kernels.hip"), os.path.join(CSRC, "zero_api.cpp")]
# host-only C++ (the optimizer half of the CPU-offloaded step), built by the
# host compiler into an object that the library links
HOST_SOURCES = [os.path.join(CSRC, "zero_host_adamw.cpp")]
LIB = os.path.join(PKG, "libzero_step.so")
OBJ_DIR = os.path.join(PKG, "_build")

HOST_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall",
    # x86-64 with AVX2 (every EPYC host of an MI355X)
    "-mavx2",
    # binary64 arithmetic exactly as written: no fused multiply-adds, no
    # fast-math; sqrt without errno so that it vectorizes (still IEEE)
    "-fno-fast-math", "-ffp-contract=off", "-fno-math-errno",
]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # exact binary32 adds and multiplies unless an fma is written out
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = ["g++", *HOST_FLAGS, "-I", CSRC, "-c", "-o", obj, src]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("g++ failed:\n" + r.stdout + r.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *SOURCES, "-x", "none", *objs,
           "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
