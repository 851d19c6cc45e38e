"""ctypes binding of libnmprobe (read-stream ceiling, one-shot read floor, copy, empty launch).

Measurement helpers only; the product calls live in sparse_matrix_vector_amd."""
import ctypes
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnmprobe.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: run __graft_entry__.build() or python measure/build.py")
        h = ctypes.CDLL(_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        h.nmp_read.argtypes = [P, I64, P, I, P]
        h.nmp_copy.argtypes = [P, P, I64, I, P]
        h.nmp_empty.argtypes = [P]
        h.nmp_read_shot.argtypes = [P, I64, P, I, P]
        for f in (h.nmp_read, h.nmp_copy, h.nmp_empty, h.nmp_read_shot):
            f.restype = I
        _lib = h
    return _lib
