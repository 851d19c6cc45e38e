"""CPU checks of the C ABI: the library loads, exports every symbol that
include/nmspmv.h declares, and rejects bad arguments before touching the GPU
(argument validation is host code; no compute call is made here)."""
import ctypes
import os
import re

import pytest

from sparse_matrix_vector_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nmspmv.h")

FAKE = 0x10000          # a 16-byte aligned address that is never dereferenced: every call below fails validation first
FAKE2 = 0x900000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for f in ("nm_pack", "nm_spmv", "nm_gemv_dense"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in L.SIGNATURES, f"binding has no signature for {name}"


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.nm_version() == 101
    for code, name in [(0, b"NM_OK"), (1, b"NM_ERR_INVALID_ARG"), (2, b"NM_ERR_BAD_SHAPE"), (3, b"NM_ERR_UNSUPPORTED"),
                       (4, b"NM_ERR_BAD_MASK"), (5, b"NM_ERR_NONFINITE"), (6, b"NM_ERR_HIP")]:
        assert lib.nm_status_string(code) == name
    assert lib.nm_status_string(99) == b"NM_ERR_UNKNOWN"


def spmv(values=FAKE, masks=FAKE, R=16, K=64, N=2, M=4, dt=0, x=FAKE2, B=1, y=FAKE2 + 0x100000):
    return L.lib().nm_spmv(values, masks, R, K, N, M, dt, x, B, y, None)


def gemv(W=FAKE, R=16, K=64, dt=0, x=FAKE2, B=1, y=FAKE2 + 0x100000):
    return L.lib().nm_gemv_dense(W, R, K, dt, x, B, y, None)


def pack(W=FAKE, keep=None, R=16, K=64, N=2, M=4, dt=0, values=FAKE2, masks=FAKE2 + 0x100000):
    return L.lib().nm_pack(W, keep, R, K, N, M, dt, values, masks, None)


@pytest.mark.parametrize("kw", [dict(K=12), dict(K=-8), dict(R=-1), dict(M=3), dict(M=16), dict(N=0), dict(N=4),
                                dict(N=8, M=8), dict(K=8 * 3, M=8, N=4) | dict(K=20), dict(B=0), dict(B=33),
                                dict(R=2 ** 31), dict(R=2 ** 31 - 1024), dict(K=2 ** 31 + 8)])
def test_spmv_bad_shape(kw):
    assert spmv(**kw) == L.NM_ERR_BAD_SHAPE


def test_spmv_unsupported_dtype():
    assert spmv(dt=2) == L.NM_ERR_UNSUPPORTED
    assert spmv(dt=-1) == L.NM_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(values=None), dict(masks=None), dict(x=None), dict(y=None),
                                dict(values=FAKE + 8), dict(masks=FAKE + 2), dict(x=FAKE2 + 4), dict(y=FAKE2 + 1),
                                dict(y=FAKE), dict(y=FAKE2 + 64)])
def test_spmv_invalid_pointer(kw):
    assert spmv(**kw) == L.NM_ERR_INVALID_ARG


def test_spmv_empty_is_ok_without_gpu():
    # R == 0: nothing to compute, no launch, pointers may be NULL.
    assert L.lib().nm_spmv(None, None, 0, 64, 2, 4, 0, FAKE2, 1, None, None) == L.NM_OK


@pytest.mark.parametrize("kw", [dict(K=12), dict(R=-1), dict(B=0), dict(B=33), dict(R=2 ** 31 - 1024)])
def test_gemv_bad_shape(kw):
    assert gemv(**kw) == L.NM_ERR_BAD_SHAPE


@pytest.mark.parametrize("kw", [dict(W=None), dict(W=FAKE + 2), dict(x=FAKE2 + 8), dict(y=None), dict(y=FAKE + 16)])
def test_gemv_invalid_pointer(kw):
    assert gemv(**kw) == L.NM_ERR_INVALID_ARG


def test_gemv_unsupported_dtype():
    assert gemv(dt=7) == L.NM_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(K=12), dict(M=2), dict(N=4), dict(N=0), dict(R=-3)])
def test_pack_bad_shape(kw):
    assert pack(**kw) == L.NM_ERR_BAD_SHAPE


@pytest.mark.parametrize("kw", [dict(W=None), dict(values=None), dict(masks=None), dict(W=FAKE + 4),
                                dict(values=FAKE2 + 2), dict(values=FAKE), dict(masks=FAKE + 32),
                                dict(keep=FAKE2 + 8)])
def test_pack_invalid_pointer(kw):
    assert pack(**kw) == L.NM_ERR_INVALID_ARG


def test_pack_empty_is_ok_without_gpu():
    assert L.lib().nm_pack(None, None, 0, 64, 2, 4, 0, None, None, None) == L.NM_OK
    assert L.lib().nm_pack(None, None, 5, 0, 2, 4, 0, None, None, None) == L.NM_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        L.lib()


def _arr(T, vals):
    return (T * len(vals))(*vals)


def test_multi_rejects_bad_count_and_null_arrays():
    lib = L.lib()
    P = ctypes.c_void_p
    v = _arr(P, [FAKE, FAKE + 0x1000])
    m = _arr(P, [FAKE + 0x2000, FAKE + 0x3000])
    R = _arr(ctypes.c_int64, [4, 4])
    y = _arr(P, [FAKE2 + 0x100000, FAKE2 + 0x200000])
    assert lib.nm_spmv_multi(0, v, m, R, 64, 2, 4, 0, FAKE2, 1, y, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_spmv_multi(5, v, m, R, 64, 2, 4, 0, FAKE2, 1, y, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_spmv_multi(2, None, m, R, 64, 2, 4, 0, FAKE2, 1, y, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_spmv_multi(2, v, m, None, 64, 2, 4, 0, FAKE2, 1, y, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_spmv_multi(2, v, m, R, 64, 2, 4, 0, FAKE2, 1, None, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_spmv_multi(2, v, m, R, 60, 2, 4, 0, FAKE2, 1, y, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_spmv_multi(2, v, m, R, 64, 2, 4, 5, FAKE2, 1, y, None) == L.NM_ERR_UNSUPPORTED
    # two outputs that overlap each other
    y_bad = _arr(P, [FAKE2 + 0x100000, FAKE2 + 0x100004])
    assert lib.nm_spmv_multi(2, v, m, R, 64, 2, 4, 0, FAKE2, 1, y_bad, None) == L.NM_ERR_INVALID_ARG
    # an output over another part's values
    y_bad = _arr(P, [FAKE2 + 0x100000, FAKE + 0x1000])
    assert lib.nm_spmv_multi(2, v, m, R, 64, 2, 4, 0, FAKE2, 1, y_bad, None) == L.NM_ERR_INVALID_ARG
    # all parts empty: nothing to do
    R0 = _arr(ctypes.c_int64, [0, 0])
    assert lib.nm_spmv_multi(2, v, m, R0, 64, 2, 4, 0, FAKE2, 1, y, None) == L.NM_OK
    Rbig = _arr(ctypes.c_int64, [2 ** 30, 2 ** 30 - 1024])          # rows stay 1024 below 2^31
    assert lib.nm_spmv_multi(2, v, m, Rbig, 64, 2, 4, 0, FAKE2, 1, y, None) == L.NM_ERR_BAD_SHAPE


def test_dense_multi_rejects_bad_arguments():
    lib = L.lib()
    P = ctypes.c_void_p
    W = _arr(P, [FAKE, FAKE + 0x10000])
    R = _arr(ctypes.c_int64, [4, 4])
    y = _arr(P, [FAKE2 + 0x100000, FAKE2 + 0x200000])
    assert lib.nm_gemv_dense_multi(0, W, R, 64, 0, FAKE2, 1, y, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_gemv_dense_multi(2, None, R, 64, 0, FAKE2, 1, y, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_gemv_dense_multi(2, W, R, 64, 0, FAKE2, 33, y, None) == L.NM_ERR_BAD_SHAPE
    Wm = _arr(P, [FAKE, FAKE + 0x10002])
    assert lib.nm_gemv_dense_multi(2, Wm, R, 64, 0, FAKE2, 1, y, None) == L.NM_ERR_INVALID_ARG


def swiglu(vg=FAKE, mg=FAKE + 0x1000, vu=FAKE + 0x2000, mu=FAKE + 0x3000, R=16, K=64, N=2, M=4, dt=0, x=FAKE2, B=1,
           h=FAKE2 + 0x100000):
    return L.lib().nm_spmv_swiglu(vg, mg, vu, mu, R, K, N, M, dt, x, B, h, None)


@pytest.mark.parametrize("kw", [dict(K=12), dict(R=-1), dict(M=3), dict(N=0), dict(N=4), dict(B=0), dict(B=33),
                                dict(R=2 ** 30 + 1), dict(R=2 ** 30 - 512)])
def test_swiglu_bad_shape(kw):
    assert swiglu(**kw) == L.NM_ERR_BAD_SHAPE


@pytest.mark.parametrize("kw", [dict(vg=None), dict(mu=None), dict(x=None), dict(h=None), dict(vu=FAKE + 0x2004),
                                dict(x=FAKE2 + 2), dict(h=FAKE2 + 0x100001), dict(h=FAKE2),
                                dict(h=FAKE + 0x2000), dict(h=FAKE + 0x3010)])
def test_swiglu_invalid_pointer(kw):
    assert swiglu(**kw) == L.NM_ERR_INVALID_ARG


def test_swiglu_dtype_and_empty():
    assert swiglu(dt=3) == L.NM_ERR_UNSUPPORTED
    assert swiglu(R=0) == L.NM_OK


def test_dense_swiglu_rejects_bad_arguments():
    lib = L.lib()
    ok_args = dict(Wg=FAKE, Wu=FAKE + 0x10000, R=16, K=64, dt=0, x=FAKE2, B=1, h=FAKE2 + 0x100000)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.nm_gemv_dense_swiglu(a["Wg"], a["Wu"], a["R"], a["K"], a["dt"], a["x"], a["B"], a["h"], None)

    assert call(K=12) == L.NM_ERR_BAD_SHAPE
    assert call(B=33) == L.NM_ERR_BAD_SHAPE
    assert call(dt=2) == L.NM_ERR_UNSUPPORTED
    assert call(Wu=None) == L.NM_ERR_INVALID_ARG
    assert call(h=FAKE + 0x10010) == L.NM_ERR_INVALID_ARG     # output over W_up
    assert call(R=0) == L.NM_OK


def test_calib_accumulate_rejects_bad_arguments():
    lib = L.lib()
    acc = lambda X=FAKE, d=None, T=4, K=64, dt=0, H=FAKE2: lib.nm_calib_accumulate(X, d, T, K, dt, H, None)  # noqa: E731
    assert acc(K=12) == L.NM_ERR_BAD_SHAPE
    assert acc(T=-1) == L.NM_ERR_BAD_SHAPE
    assert acc(K=65544) == L.NM_ERR_BAD_SHAPE
    assert acc(dt=7) == L.NM_ERR_UNSUPPORTED
    assert acc(X=None) == L.NM_ERR_INVALID_ARG
    assert acc(X=FAKE + 8) == L.NM_ERR_INVALID_ARG
    assert acc(H=FAKE2 + 2) == L.NM_ERR_INVALID_ARG
    assert acc(H=FAKE + 0x100) == L.NM_ERR_INVALID_ARG          # H over X
    assert acc(d=FAKE2 + 0x40) == L.NM_ERR_INVALID_ARG          # decode flags inside H
    assert acc(T=0) == L.NM_OK and acc(K=0) == L.NM_OK


def test_calib_keep_mask_rejects_bad_arguments():
    lib = L.lib()

    def keep(W=FAKE, h=FAKE2, hs=1, R=4, K=64, N=2, M=4, dt=0, out=FAKE2 + 0x100000):
        return lib.nm_calib_keep_mask(W, h, hs, R, K, N, M, dt, out, None)

    assert keep(K=12) == L.NM_ERR_BAD_SHAPE
    assert keep(N=4) == L.NM_ERR_BAD_SHAPE
    assert keep(M=5) == L.NM_ERR_BAD_SHAPE
    assert keep(hs=0) == L.NM_ERR_BAD_SHAPE
    assert keep(dt=9) == L.NM_ERR_UNSUPPORTED
    assert keep(W=FAKE + 4) == L.NM_ERR_INVALID_ARG
    assert keep(out=FAKE2 + 0x100004) == L.NM_ERR_INVALID_ARG
    assert keep(h=None) == L.NM_ERR_INVALID_ARG
    assert keep(out=FAKE) == L.NM_ERR_INVALID_ARG               # keep over W
    assert keep(R=0) == L.NM_OK


def test_hybrid_calls_reject_bad_arguments():
    lib = L.lib()
    # row loss
    assert lib.nm_hybrid_row_loss(FAKE, None, None, 0, 4, 12, 2, 4, 0, FAKE2, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_hybrid_row_loss(FAKE, None, FAKE2 + 0x1000, 0, 4, 64, 2, 4, 0, FAKE2, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_hybrid_row_loss(FAKE, None, None, 0, 4, 64, 2, 4, 0, FAKE2 + 4, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_hybrid_row_loss(FAKE, None, None, 0, 4, 64, 2, 4, 0, FAKE + 8, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_hybrid_row_loss(FAKE, None, None, 0, 4, 64, 2, 4, 5, FAKE2, None) == L.NM_ERR_UNSUPPORTED
    assert lib.nm_hybrid_row_loss(FAKE, None, None, 0, 0, 64, 2, 4, 0, FAKE2, None) == L.NM_OK
    # row choice
    assert lib.nm_hybrid_select_rows(FAKE, 10, 11, FAKE2, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_hybrid_select_rows(FAKE, 10, -1, FAKE2, None) == L.NM_ERR_BAD_SHAPE
    assert lib.nm_hybrid_select_rows(FAKE + 4, 10, 2, FAKE2, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_hybrid_select_rows(FAKE, 10, 2, FAKE + 16, None) == L.NM_ERR_INVALID_ARG     # flags over loss
    assert lib.nm_hybrid_select_rows(FAKE, 0, 0, FAKE2, None) == L.NM_OK
    # pack: outputs must not overlap each other or the inputs
    P = 0x4000000
    args = dict(W=P, keep=None, flags=P + 0x100000, nd=2, R=8, K=64, N=2, M=4, dt=0, values=P + 0x200000,
                masks=P + 0x300000, Wd=P + 0x400000, rs=P + 0x500000, rd=P + 0x600000)

    def pack(**kw):
        a = dict(args, **kw)
        return lib.nm_hybrid_pack(a["W"], a["keep"], a["flags"], a["nd"], a["R"], a["K"], a["N"], a["M"], a["dt"],
                                  a["values"], a["masks"], a["Wd"], a["rs"], a["rd"], None)

    assert pack(nd=9) == L.NM_ERR_BAD_SHAPE
    assert pack(K=12) == L.NM_ERR_BAD_SHAPE
    assert pack(values=P + 0x200008) == L.NM_ERR_INVALID_ARG
    assert pack(rd=P + 0x600002) == L.NM_ERR_INVALID_ARG
    assert pack(Wd=P + 0x200000) == L.NM_ERR_INVALID_ARG            # W_dense over values
    assert pack(rs=P + 0x10) == L.NM_ERR_INVALID_ARG                # rows over W
    assert pack(R=0, nd=0) == L.NM_OK
    # product
    def spmv(**kw):
        a = dict(v=P, m=P + 0x100000, rs=P + 0x200000, Wd=P + 0x300000, rd=P + 0x400000, nd=2, R=8, K=64, N=2, M=4,
                 dt=0, x=P + 0x500000, B=1, y=P + 0x600000)
        a.update(kw)
        return lib.nm_spmv_hybrid(a["v"], a["m"], a["rs"], a["Wd"], a["rd"], a["nd"], a["R"], a["K"], a["N"], a["M"],
                                  a["dt"], a["x"], a["B"], a["y"], None)

    assert spmv(B=33) == L.NM_ERR_BAD_SHAPE
    assert spmv(nd=9) == L.NM_ERR_BAD_SHAPE
    assert spmv(y=P + 0x500000) == L.NM_ERR_INVALID_ARG              # y over x
    assert spmv(y=P + 0x400004) == L.NM_ERR_INVALID_ARG              # y over rows_dense
    assert spmv(rs=P + 0x200002) == L.NM_ERR_INVALID_ARG
    assert spmv(R=0, nd=0) == L.NM_OK


def test_workspace_calls_check_the_workspace():
    lib = L.lib()
    P = ctypes.c_void_p
    need = lib.nm_workspace_bytes()
    assert need >= 16 << 20
    v = _arr(P, [FAKE])
    m = _arr(P, [FAKE + 0x1000])
    R = _arr(ctypes.c_int64, [4])
    y = _arr(P, [FAKE2 + 0x100000])
    WS = 0x40000000                                   # 256-byte aligned, far from every buffer above
    ws_call = lambda ws, nb, R=R: lib.nm_spmv_multi_ws(1, v, m, R, 64, 2, 4, 0, FAKE2, 8, y, ws, nb, None)  # noqa: E731
    assert ws_call(WS, need - 1) == L.NM_ERR_INVALID_ARG            # too small
    assert ws_call(WS + 16, need) == L.NM_ERR_INVALID_ARG           # misaligned
    assert ws_call(FAKE2 - 256, need) == L.NM_ERR_INVALID_ARG       # over x
    y_far = _arr(P, [0x50000000])
    assert lib.nm_spmv_multi_ws(1, v, m, R, 64, 2, 4, 0, FAKE2, 8, y_far, 0x50000000 - need + 256, need,
                                None) == L.NM_ERR_INVALID_ARG                       # over y
    assert lib.nm_spmv_multi_ws(1, v, m, R, 64, 2, 4, 0, FAKE2, 8, y, FAKE - 256, need,
                                None) == L.NM_ERR_INVALID_ARG                       # over the values
    R0 = _arr(ctypes.c_int64, [0])
    assert ws_call(WS, need, R0) == L.NM_OK                          # nothing to do
    assert ws_call(None, 0, R0) == L.NM_OK                           # no workspace: the plain call
    Wd = _arr(P, [FAKE])
    assert lib.nm_gemv_dense_multi_ws(1, Wd, R, 64, 0, FAKE2, 8, y, WS, need - 1, None) == L.NM_ERR_INVALID_ARG
    assert lib.nm_gemv_dense_multi_ws(1, Wd, R0, 64, 0, FAKE2, 8, y, WS, need, None) == L.NM_OK
