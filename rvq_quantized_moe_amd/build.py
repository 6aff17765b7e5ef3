"""Builds librvq.so (the C-ABI library) in-tree with hipcc for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librvq.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "chunk.hip"), os.path.join(CSRC, "verify.hip"),
           os.path.join(CSRC, "encode.hip"), os.path.join(CSRC, "scratch.hip"),
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "pool.cpp")]
HEADERS = [os.path.join(CSRC, "device.hpp"), os.path.join(CSRC, "launch.hpp"), os.path.join(ROOT, "include", "rvq.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # packed fp32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(verbose=False):
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


def is_stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
