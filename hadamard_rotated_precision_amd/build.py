"""Build libhq.so (the gfx950 HIP kernels and the C ABI of include/hq.h) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhq.so")

SOURCES = ["hq_rotate.hip", "hq_prologue.hip", "hq_gemm.hip", "hq_static.hip", "hq_lss.hip", "hq_api.cpp",
           "hq_profile.cpp"]

# -packed-fp32-ops: hipcc forms packed fp32 ops from plain float code; keep them out.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
             "-I" + os.path.join(ROOT, "include")]


def build(verbose=False, jobs=None):
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc"] + HIP_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
        objs.append(obj)
    for cmd, p in procs:
        if p.wait() != 0:
            raise RuntimeError("compile failed: " + " ".join(cmd))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
