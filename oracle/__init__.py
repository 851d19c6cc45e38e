"""CPU oracle for N:M sparse matrix-vector products.

TEST INFRASTRUCTURE ONLY: importable from the test suite, the smoke check and
the benchmark's CPU-baseline leg, never from the product path.  It shares no
code with the GPU library; the plain-C core is ``nm_oracle.c`` and this module
only marshals numpy arrays into it and adds the acceptance rule.

Sources (see ``nm_oracle.c`` for the readings of open points):
  * SparseDecoding abstract (humanity-list story page, "Abstract"): the hot
    operation is an N:M sparse matrix-vector product over a pruned weight,
    indexed by a bitmask and walked with a fixed step.
  * bedrocknews arXiv 2610.12327v1 article: N:M keeps a fixed ratio inside
    every small block; the product is a sparse matrix times a single vector.

Every function below is pinned by the CPU tests (``tests/test_oracle_*.py``)
against closed forms, brute force, exhaustive format checks and hand-worked
fixtures under ``tests/golden/``.
"""
import ctypes
import math
import os

import numpy as np

FP16, BF16 = 0, 1
DTYPES = {"fp16": FP16, "bf16": BF16}

OK, BAD_ARG, BAD_SHAPE, BAD_MASK, NONFINITE = 0, 1, 2, 4, 5
_NAMES = {OK: "OK", BAD_ARG: "BAD_ARG", BAD_SHAPE: "BAD_SHAPE", BAD_MASK: "BAD_MASK", NONFINITE: "NONFINITE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBS = {}


class OracleError(RuntimeError):
    def __init__(self, status):
        super().__init__(f"oracle status {_NAMES.get(status, status)}")
        self.status = status


_CURRENT = [None]


def _lib():
    if _CURRENT[0] is None:
        path = os.path.join(_HERE, "liboracle.so")
        src = os.path.join(_HERE, "nm_oracle.c")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            from . import build as _build
            _build.build()
        _CURRENT[0] = _load(path)
    return _CURRENT[0]


def use_library(path):
    """Point the module at another build of nm_oracle.c (the CPU tests use
    this to plant mistakes in a copy and check that the pins catch them).
    ``None`` returns to the default build.  Returns the previous library."""
    prev = _CURRENT[0]
    _CURRENT[0] = None if path is None else _load(path)
    return prev


def _load(path):
    if path not in _LIBS:
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.orc_pack.argtypes = [P, P, I64, I64, I, I, I, P, P]
        lib.orc_expand.argtypes = [P, P, I64, I64, I, I, P]
        lib.orc_spmv_rows.argtypes = [P, P, I64, I64, I, I, I, P, I, I64, I64, P, P]
        lib.orc_gemv_rows.argtypes = [P, I64, I64, I, P, I, I64, I64, P, P]
        lib.orc_round_array.argtypes = [P, I64, I, P]
        lib.orc_decode_array.argtypes = [P, I64, I, P]
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_swiglu.argtypes = [P, P, I64, P]
        lib.orc_calib_accumulate.argtypes = [P, P, I64, I64, I, P, P]
        lib.orc_calib_keep.argtypes = [P, P, I64, I64, I, I, I, P]
        lib.orc_hybrid_row_loss.argtypes = [P, P, P, I64, I64, I, I, I, P]
        lib.orc_hybrid_select.argtypes = [P, I64, I64, P]
        for f in ("orc_pack", "orc_expand", "orc_spmv_rows", "orc_gemv_rows"):
            getattr(lib, f).restype = ctypes.c_int
        lib.orc_round_array.restype = None
        lib.orc_decode_array.restype = None
        _LIBS[path] = lib
    return _LIBS[path]


def _dt(dtype):
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16) if a.dtype.itemsize == 2 else a
    assert a.dtype == np.uint16, a.dtype
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(bits, dtype):
    """16-bit encodings -> exact float64 values."""
    bits = _u16(bits)
    out = np.empty(bits.shape, np.float64)
    _lib().orc_decode_array(_ptr(bits), bits.size, _dt(dtype), _ptr(out))
    return out


def round_to(y, dtype):
    """float64 -> 16-bit encodings, round to nearest even, overflow to inf."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(y.shape, np.uint16)
    _lib().orc_round_array(_ptr(y), y.size, _dt(dtype), _ptr(out))
    return out


def pack(W, keep, n, m, dtype):
    """W [R][K] 16-bit encodings (+ keep [R][K] nonzero=keep, or None for
    top-n by magnitude, lowest index first) -> (values [R][K*n/m] uint16,
    masks [R][K/8] uint8)."""
    W = _u16(W)
    R, K = W.shape
    if keep is not None:
        keep = np.ascontiguousarray(keep).view(np.uint8) if keep.dtype == np.bool_ else np.ascontiguousarray(keep, np.uint8)
        assert keep.shape == W.shape
    vals = np.zeros((R, K * n // m if K % m == 0 else 0), np.uint16)
    masks = np.zeros((R, K // 8), np.uint8)
    st = _lib().orc_pack(_ptr(W), _ptr(keep), R, K, n, m, _dt(dtype), _ptr(vals), _ptr(masks))
    if st != OK:
        raise OracleError(st)
    return vals, masks


def expand(values, masks, K, n, m):
    """Packed (values, masks) -> dense pruned 16-bit matrix [R][K]."""
    values = _u16(values)
    masks = np.ascontiguousarray(masks, np.uint8)
    R = masks.shape[0]
    out = np.empty((R, K), np.uint16)
    st = _lib().orc_expand(_ptr(values), _ptr(masks), R, K, n, m, _ptr(out))
    if st != OK:
        raise OracleError(st)
    return out


def spmv(values, masks, K, n, m, dtype, x, rows=None):
    """Sparse product in float64.  x [B][K] 16-bit encodings.  Returns
    (y [B][R'], A [B][R']) with A = sum |w*x| over the kept terms.  ``rows``
    (a (r0, r1) range) restricts the work to those rows."""
    values, x = _u16(values), _u16(np.atleast_2d(x))
    masks = np.ascontiguousarray(masks, np.uint8)
    R = masks.shape[0]
    B = x.shape[0]
    assert x.shape[1] == K
    r0, r1 = (0, R) if rows is None else rows
    y = np.zeros((B, R), np.float64)
    A = np.zeros((B, R), np.float64)
    st = _lib().orc_spmv_rows(_ptr(values), _ptr(masks), R, K, n, m, _dt(dtype), _ptr(x), B, r0, r1, _ptr(y), _ptr(A))
    if st != OK:
        raise OracleError(st)
    return y[:, r0:r1].copy(), A[:, r0:r1].copy()


def gemv(W, dtype, x, rows=None):
    """Dense product in float64.  W [R][K], x [B][K] 16-bit encodings."""
    W, x = _u16(W), _u16(np.atleast_2d(x))
    R, K = W.shape
    B = x.shape[0]
    r0, r1 = (0, R) if rows is None else rows
    y = np.zeros((B, R), np.float64)
    A = np.zeros((B, R), np.float64)
    st = _lib().orc_gemv_rows(_ptr(W), R, K, _dt(dtype), _ptr(x), B, r0, r1, _ptr(y), _ptr(A))
    if st != OK:
        raise OracleError(st)
    return y[:, r0:r1].copy(), A[:, r0:r1].copy()


def silu(t):
    """SiLU(t) = t / (1 + e^-t) of one float, in double."""
    return float(_lib().orc_silu(float(t)))


def swiglu(g, u):
    """h = SiLU(g) * u elementwise, in double (g, u: the exact sums of the
    gate and up products)."""
    g = np.ascontiguousarray(g, np.float64)
    u = np.ascontiguousarray(u, np.float64)
    assert g.shape == u.shape
    h = np.zeros(g.shape, np.float64)
    _lib().orc_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def calib_accumulate(X, dtype, decode=None, H=None, A=None):
    """Decoding-aware calibration statistics in double: H += sum over decode
    rows t of x_t x_t^T (X [T][K] 16-bit encodings; decode [T] bytes, nonzero =
    decode step, None = all rows), and A += the sum of |x_ti x_tj|.  Returns
    (H, A), each [K][K] float64."""
    X = _u16(np.atleast_2d(X))
    T, K = X.shape
    H = np.zeros((K, K), np.float64) if H is None else np.ascontiguousarray(H, np.float64).copy()
    A = np.zeros((K, K), np.float64) if A is None else np.ascontiguousarray(A, np.float64).copy()
    d = None
    if decode is not None:
        d = np.ascontiguousarray(decode, np.uint8)
        assert d.shape == (T,)
    st = _lib().orc_calib_accumulate(_ptr(X), None if d is None else _ptr(d), T, K, _dt(dtype), _ptr(H), _ptr(A))
    if st != OK:
        raise OracleError(st)
    return H, A


def calib_keep(W, hdiag, n, m, dtype):
    """Keep-mask [R][K] (uint8, 1 = keep) of the n columns per m-group with the
    largest w^2 * hdiag[c], lower column on ties.  hdiag: float32 values (the
    diagonal the GPU reads), used exactly."""
    W = _u16(W)
    R, K = W.shape
    h = np.ascontiguousarray(np.asarray(hdiag, np.float32).astype(np.float64))
    assert h.shape == (K,)
    keep = np.zeros((R, K), np.uint8)
    st = _lib().orc_calib_keep(_ptr(W), _ptr(h), R, K, n, m, _dt(dtype), _ptr(keep))
    if st != OK:
        raise OracleError(st)
    return keep


def hybrid_row_loss(W, n, m, dtype, keep=None, h=None):
    """Per-row pruning loss L_r = sum over pruned columns of w^2 h[c] (h: float32
    values used exactly, or None for 1), pruned by the keep-mask or by top-n
    magnitude.  Returns float64 [R]."""
    W = _u16(W)
    R, K = W.shape
    kp = None if keep is None else np.ascontiguousarray(keep, np.uint8)
    hv = None if h is None else np.ascontiguousarray(np.asarray(h, np.float32).astype(np.float64))
    loss = np.zeros(R, np.float64)
    st = _lib().orc_hybrid_row_loss(_ptr(W), None if kp is None else _ptr(kp), None if hv is None else _ptr(hv),
                                    R, K, n, m, _dt(dtype), _ptr(loss))
    if st != OK:
        raise OracleError(st)
    return loss


def hybrid_select(loss, n_dense):
    """uint8 [R] flags of the n_dense rows of largest loss (NaN lowest, lower row first)."""
    loss = np.ascontiguousarray(loss, np.float64)
    flags = np.zeros(loss.shape[0], np.uint8)
    st = _lib().orc_hybrid_select(_ptr(loss), loss.shape[0], n_dense, _ptr(flags))
    if st != OK:
        raise OracleError(st)
    return flags


def hybrid_spmv(W, flags, n, m, dtype, x, keep=None):
    """The hybrid matrix's product: rows flagged dense use W as is, the others
    its n:m pruned form (keep-mask or top-n).  Returns (y, A) [B][R] in double."""
    W = _u16(W)
    R, K = W.shape
    x = _u16(np.atleast_2d(x))
    d = np.asarray(flags, bool)
    y = np.zeros((x.shape[0], R))
    A = np.zeros((x.shape[0], R))
    if (~d).any():
        v, mk = pack(W[~d], None if keep is None else np.asarray(keep)[~d], n, m, dtype)
        y[:, ~d], A[:, ~d] = spmv(v, mk, K, n, m, dtype, x)
    if d.any():
        y[:, d], A[:, d] = gemv(W[d], dtype, x)
    return y, A


# ---- acceptance rule ------------------------------------------------------

_FMT = {FP16: (10, -14), BF16: (7, -126)}   # (fraction bits, min normal exponent)
REL_TOL = 2e-3


def ulp(t, dtype):
    """Gap of the 16-bit format at |t|: 2^(max(floor(log2|t|), emin) - fbits);
    at t == 0 the smallest subnormal."""
    fbits, emin = _FMT[_dt(dtype)]
    t = np.abs(np.asarray(t, np.float64))
    _, e = np.frexp(t)                        # t = f * 2^e, f in [0.5, 1)
    e = np.where(t == 0, emin, np.maximum(e - 1, emin))
    return np.ldexp(1.0, e - fbits)


def tolerance(y_ref, A, dtype):
    """Per-element bound: 2e-3 * sum|w*x| + one ulp of the output format at y_ref."""
    return REL_TOL * np.asarray(A, np.float64) + ulp(y_ref, dtype)


def check(y_bits, y_ref, A, dtype):
    """Return (ok, worst_ratio, index) for a GPU result given as 16-bit
    encodings against the float64 reference."""
    got = decode(y_bits, dtype)
    err = np.abs(got - y_ref)
    tol = tolerance(y_ref, A, dtype)
    ratio = np.where(np.isfinite(err), err / tol, np.inf)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    worst = float(ratio[idx]) if ratio.size else 0.0
    return bool(np.all(err <= tol)), worst, idx


def max_terms_bound(n_terms):
    """gamma_{n-1} = (n-1)u / (1 - (n-1)u), u = 2^-24: the worst relative
    error (against sum|terms|) of any fp32 summation order of n exact terms."""
    u = math.ldexp(1.0, -24)
    k = n_terms - 1
    return k * u / (1 - k * u)


# SiLU is Lipschitz with constant max|SiLU'| = 1.0998 (at t ~ 2.40); 1.1 bounds it.
SILU_LIP = 1.1
# Evaluation of SiLU(g) * u from the fp32 sums (a few roundings in double, then
# one to fp32 before the 16-bit rounding): 2^-24 relative and change; 1e-5
# covers it with a wide margin.
GLU_EVAL_REL = 1e-5


def swiglu_tolerance(g_ref, u_ref, Ag, Au, dtype, exact_sums=False):
    """Bound on |h_gpu - h_ref| for h = SiLU(g) * u computed from fp32 sums g,
    u whose own errors obey the product rule (|e| <= 2e-3 * sum|w*x|; zero when
    the sums are exact, e.g. integer-valued operands):
        |SiLU(g)u - SiLU(g_ref)u_ref| <= 1.1 e_g (|u_ref| + e_u) + |SiLU(g_ref)| e_u
    plus the fp32 evaluation error and one ulp of the output format."""
    g_ref, u_ref = np.asarray(g_ref, np.float64), np.asarray(u_ref, np.float64)
    eg = np.zeros_like(g_ref) if exact_sums else REL_TOL * np.asarray(Ag, np.float64)
    eu = np.zeros_like(u_ref) if exact_sums else REL_TOL * np.asarray(Au, np.float64)
    h_ref = swiglu(g_ref, u_ref)
    s_ref = np.abs(swiglu(g_ref, np.ones_like(g_ref)))
    return (SILU_LIP * eg * (np.abs(u_ref) + eu) + s_ref * eu + GLU_EVAL_REL * np.abs(h_ref) + ulp(h_ref, dtype))


def check_swiglu(h_bits, g_ref, u_ref, Ag, Au, dtype, exact_sums=False):
    """(ok, worst_ratio, index) for a GPU h (16-bit encodings) against
    SiLU(g_ref) * u_ref."""
    got = decode(h_bits, dtype)
    h_ref = swiglu(g_ref, u_ref)
    err = np.abs(got - h_ref)
    tol = swiglu_tolerance(g_ref, u_ref, Ag, Au, dtype, exact_sums)
    ratio = np.where(np.isfinite(err), err / tol, np.inf)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    worst = float(ratio[idx]) if ratio.size else 0.0
    return bool(np.all(err <= tol)), worst, idx


def check_calib(H_gpu, H_ref, A, H0=None):
    """(ok, worst_ratio, index) for a GPU fp32 H against the double H_ref: any
    fp32 summation order of T exact products (plus the prior contents H0)
    errs by at most gamma_T * (sum|x_i x_j| + |H0|) (gamma_T < 2e-3 for T up to
    ~33000); one fp32 ulp at H_ref covers the last rounding."""
    H_gpu = np.asarray(H_gpu, np.float64)
    base = np.asarray(A, np.float64) + (0.0 if H0 is None else np.abs(np.asarray(H0, np.float64)))
    ulp32 = np.spacing(np.abs(H_ref).astype(np.float32)).astype(np.float64)
    tol = REL_TOL * base + ulp32
    err = np.abs(H_gpu - H_ref)
    ratio = np.where(np.isfinite(err), err / tol, np.inf)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    worst = float(ratio[idx]) if ratio.size else 0.0
    return bool(np.all(err <= tol)), worst, idx
