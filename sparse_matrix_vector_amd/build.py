"""Compile libnmspmv.so (HIP, gfx950) in-tree with hipcc.

Always recompiles: the caller asked for a build.  The shared library lands
next to this file so it travels with the source tree.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(HERE, "csrc", "nmapi.cpp"), os.path.join(HERE, "csrc", "nmspmv.hip"),
       os.path.join(HERE, "csrc", "nmcalib.hip")]
LIB = os.path.join(HERE, "libnmspmv.so")
# (sources, library): the product library
TARGETS = [(SRC, LIB)]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnmspmv)")


def build(verbose: bool = False) -> str:
    for src, lib in TARGETS:
        build_one(src, lib, verbose)
    return LIB


def build_one(src, lib, verbose=False):
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed-fp32 instructions stay off (the compiler would otherwise form them from float code)
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-fno-gpu-rdc", "-Wall", "-Wno-unused-result",
           "-I", os.path.join(ROOT, "include"), *src, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
