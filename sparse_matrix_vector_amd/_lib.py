"""ctypes binding of libnmspmv (include/nmspmv.h).

Argument marshalling only: every step of the product runs in the HIP library.
There is no fallback: if ``libnmspmv.so`` is missing the first call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnmspmv.so")

NM_OK, NM_ERR_INVALID_ARG, NM_ERR_BAD_SHAPE, NM_ERR_UNSUPPORTED = 0, 1, 2, 3
NM_ERR_BAD_MASK, NM_ERR_NONFINITE, NM_ERR_HIP = 4, 5, 6
NM_FP16, NM_BF16 = 0, 1

# Every symbol the header declares, with its ctypes signature.
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "nm_pack": (_I, [_P, _P, _I64, _I64, _I, _I, _I, _P, _P, _P]),
    "nm_spmv": (_I, [_P, _P, _I64, _I64, _I, _I, _I, _P, _I, _P, _P]),
    "nm_gemv_dense": (_I, [_P, _I64, _I64, _I, _P, _I, _P, _P]),
    "nm_spmv_multi": (_I, [_I, _P, _P, _P, _I64, _I, _I, _I, _P, _I, _P, _P]),
    "nm_gemv_dense_multi": (_I, [_I, _P, _P, _I64, _I, _P, _I, _P, _P]),
    "nm_workspace_bytes": (_I64, []),
    "nm_spmv_multi_ws": (_I, [_I, _P, _P, _P, _I64, _I, _I, _I, _P, _I, _P, _P, _I64, _P]),
    "nm_gemv_dense_multi_ws": (_I, [_I, _P, _P, _I64, _I, _P, _I, _P, _P, _I64, _P]),
    "nm_spmv_multi_noalloc": (_I, [_I, _P, _P, _P, _I64, _I, _I, _I, _P, _I, _P, _P]),
    "nm_spmv_swiglu": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, _I, _P, _I, _P, _P]),
    "nm_gemv_dense_swiglu": (_I, [_P, _P, _I64, _I64, _I, _P, _I, _P, _P]),
    "nm_calib_accumulate": (_I, [_P, _P, _I64, _I64, _I, _P, _P]),
    "nm_calib_keep_mask": (_I, [_P, _P, _I64, _I64, _I64, _I, _I, _I, _P, _P]),
    "nm_hybrid_row_loss": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _P, _P]),
    "nm_hybrid_select_rows": (_I, [_P, _I64, _I64, _P, _P]),
    "nm_hybrid_pack": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "nm_spmv_hybrid": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _I, _P, _I, _P, _P]),
    "nm_status_string": (ctypes.c_char_p, [_I]),
    "nm_version": (_I, []),
}

_lib = None


class NmError(RuntimeError):
    """A libnmspmv call returned a status other than NM_OK."""

    def __init__(self, func, status):
        name = lib().nm_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{func} failed: {name}")
        self.status = status


def lib():
    """Load libnmspmv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python sparse_matrix_vector_amd/build.py")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != NM_OK:
        raise NmError(name, st)
    return st
