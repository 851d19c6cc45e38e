"""Compile libnmprobe.so (the measurement probes, HIP, gfx950) in-tree.

Always recompiles; uses the product library's compiler settings.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

LIB = os.path.join(HERE, "libnmprobe.so")


def build(verbose: bool = False) -> str:
    from sparse_matrix_vector_amd import build as product_build
    return product_build.build_one([os.path.join(HERE, "nmprobe.hip")], LIB, verbose)


if __name__ == "__main__":
    build(verbose=True)
