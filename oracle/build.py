"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure only: the GPU library never links or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile nm_oracle.c with gcc.  No fast-math, no vector intrinsics: the
    floating-point sums keep the source's ascending order."""
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
