"""libnmspmv for MI355X: N:M semi-structured sparse matrix-vector products.

Python face of the C ABI in ``include/nmspmv.h``.  Tensors are torch CUDA
(HIP) tensors; torch supplies device memory and the current stream, and every
step of the computation runs in the HIP kernels of ``libnmspmv.so``.

    values, masks = pack(W, keep=None, n=2, m=4)   # offline: prune + pack
    y = spmv(values, masks, x, n=2, m=4)           # per token: y = W_sparse x
    y = gemv_dense(W, x)                           # dense baseline
    h = spmv_swiglu((vg, mg), (vu, mu), x)         # SiLU(W_gate x) * (W_up x)
    H = calib_accumulate(X, decode)                # decoding-aware calibration
    keep = calib_keep_mask(W, H, n=2, m=4)         # -> pack(W, keep, 2, 4)
    hyb = hybrid_pack(W, hybrid_select_rows(hybrid_row_loss(W), n_dense))
    y = spmv_hybrid(hyb, x)                        # sparse rows + dense rows
    ys = spmv_multi(parts, x, ws=workspace())      # K-split plan for batches on few rows
"""
import ctypes

import torch

from ._lib import (NM_BF16, NM_ERR_BAD_MASK, NM_ERR_BAD_SHAPE, NM_ERR_HIP, NM_ERR_INVALID_ARG,  # noqa: F401
                   NM_ERR_NONFINITE, NM_ERR_UNSUPPORTED, NM_FP16, NM_OK, NmError, call, lib)

__all__ = ["pack", "spmv", "spmv_multi", "spmv_swiglu", "gemv_dense", "gemv_dense_multi", "gemv_dense_swiglu",
           "calib_accumulate", "calib_keep_mask", "hybrid_row_loss", "hybrid_select_rows", "hybrid_pack", "spmv_hybrid",
           "Hybrid", "NmError", "dtype_code", "stream_handle", "workspace"]

_DT = {torch.float16: NM_FP16, torch.bfloat16: NM_BF16}


def dtype_code(dtype):
    if dtype not in _DT:
        raise TypeError(f"libnmspmv supports float16 and bfloat16, not {dtype}")
    return _DT[dtype]


def stream_handle(stream=None):
    """hipStream_t of ``stream`` (default: torch's current stream) for the C ABI."""
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def pack(W, keep=None, n=2, m=4, stream=None):
    """Prune W [R][K] to n:m and pack it.  ``keep`` is a bool/uint8 tensor of
    W's shape (nonzero = keep, exactly n per group) or None for top-n by
    magnitude (lower column wins ties).  Returns (values [R][K*n/m] in W's
    dtype, masks [R][K/8] uint8)."""
    _dev(W, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [R][K]")
    R, K = W.shape
    kp = None
    if keep is not None:
        _dev(keep, "keep")
        if keep.shape != W.shape or keep.dtype not in (torch.bool, torch.uint8):
            raise ValueError("keep must be a bool/uint8 tensor shaped like W")
        kp = keep.data_ptr()
    if m <= 0 or K % m:
        raise ValueError("K must be a multiple of m")
    values = torch.empty((R, K // m * n), dtype=W.dtype, device=W.device)
    masks = torch.empty((R, K // 8), dtype=torch.uint8, device=W.device)
    call("nm_pack", W.data_ptr(), kp, R, K, n, m, dtype_code(W.dtype), values.data_ptr(), masks.data_ptr(),
         stream_handle(stream))
    return values, masks


def spmv(values, masks, x, n=2, m=4, out=None, stream=None):
    """y = W_sparse x.  x is [K] or [B][K] (B <= 32); returns [R] or [B][R]."""
    _dev(values, "values"), _dev(masks, "masks"), _dev(x, "x")
    R = masks.shape[0]
    K = masks.shape[1] * 8
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    B = x2.shape[0]
    if x2.shape[1] != K or x.dtype != values.dtype:
        raise ValueError("x must be [B][K] in the values' dtype")
    if values.shape != (R, K // m * n):
        raise ValueError("values shape does not match masks and n:m")
    y = torch.empty((B, R), dtype=values.dtype, device=values.device) if out is None else _dev(out, "out")
    call("nm_spmv", values.data_ptr(), masks.data_ptr(), R, K, n, m, dtype_code(values.dtype), x2.data_ptr(), B,
         y.data_ptr(), stream_handle(stream))
    return y[0] if squeeze else y


def gemv_dense(W, x, out=None, stream=None):
    """Dense baseline y = W x.  x is [K] or [B][K]; returns [R] or [B][R]."""
    _dev(W, "W"), _dev(x, "x")
    R, K = W.shape
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    B = x2.shape[0]
    if x2.shape[1] != K or x.dtype != W.dtype:
        raise ValueError("x must be [B][K] in W's dtype")
    y = torch.empty((B, R), dtype=W.dtype, device=W.device) if out is None else _dev(out, "out")
    call("nm_gemv_dense", W.data_ptr(), R, K, dtype_code(W.dtype), x2.data_ptr(), B, y.data_ptr(),
         stream_handle(stream))
    return y[0] if squeeze else y


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return arr


def workspace(device="cuda"):
    """A zero-filled K-split workspace (nm_workspace_bytes() bytes) for
    spmv_multi / gemv_dense_multi on `device`; give each stream its own."""
    nbytes = int(lib().nm_workspace_bytes())
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _ws_args(ws):
    if ws is None:
        return None, 0
    _dev(ws, "workspace")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def spmv_multi(parts, x, n=2, m=4, stream=None, ws=None):
    """One launch for several packed matrices sharing x (e.g. q, k, v).
    ``parts`` is a list of (values, masks); returns a list of y [B][R_i]
    (or [R_i] for a 1-D x).  ``ws``: a workspace() for the K-split plan of
    batched products on few rows (nm_spmv_multi_ws), or None."""
    if not 1 <= len(parts) <= 4:
        raise ValueError("1 to 4 parts")
    _dev(x, "x")
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    B, K = x2.shape
    ys, Rs = [], []
    for values, masks in parts:
        _dev(values, "values"), _dev(masks, "masks")
        R = masks.shape[0]
        if masks.shape[1] * 8 != K or values.shape != (R, K // m * n) or values.dtype != x.dtype:
            raise ValueError("part shapes do not match x and n:m")
        ys.append(torch.empty((B, R), dtype=x.dtype, device=x.device))
        Rs.append(R)
    args = (len(parts), _ptr_array([v.data_ptr() for v, _ in parts]), _ptr_array([mk.data_ptr() for _, mk in parts]),
            (ctypes.c_int64 * len(parts))(*Rs), K, n, m, dtype_code(x.dtype), x2.data_ptr(), B,
            _ptr_array([y.data_ptr() for y in ys]))
    if ws is None:
        call("nm_spmv_multi", *args, stream_handle(stream))
    else:
        call("nm_spmv_multi_ws", *args, *_ws_args(ws), stream_handle(stream))
    return [y[0] for y in ys] if squeeze else ys


def gemv_dense_multi(Ws, x, stream=None, ws=None):
    """Dense baseline of spmv_multi: one launch for several W sharing x
    (``ws`` as in spmv_multi)."""
    if not 1 <= len(Ws) <= 4:
        raise ValueError("1 to 4 matrices")
    _dev(x, "x")
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    B, K = x2.shape
    ys = []
    for W in Ws:
        _dev(W, "W")
        if W.shape[1] != K or W.dtype != x.dtype:
            raise ValueError("W shapes do not match x")
        ys.append(torch.empty((B, W.shape[0]), dtype=x.dtype, device=x.device))
    args = (len(Ws), _ptr_array([W.data_ptr() for W in Ws]), (ctypes.c_int64 * len(Ws))(*[W.shape[0] for W in Ws]), K,
            dtype_code(x.dtype), x2.data_ptr(), B, _ptr_array([y.data_ptr() for y in ys]))
    if ws is None:
        call("nm_gemv_dense_multi", *args, stream_handle(stream))
    else:
        call("nm_gemv_dense_multi_ws", *args, *_ws_args(ws), stream_handle(stream))
    return [y[0] for y in ys] if squeeze else ys


def _x2(x):
    _dev(x, "x")
    squeeze = x.dim() == 1
    return (x.unsqueeze(0) if squeeze else x), squeeze


def spmv_swiglu(gate, up, x, n=2, m=4, out=None, stream=None):
    """h = SiLU(W_gate x) * (W_up x) in one launch.  ``gate`` and ``up`` are
    (values, masks) pairs packed with the same n:m; x is [K] or [B][K];
    returns [R] or [B][R]."""
    (vg, mg), (vu, mu) = gate, up
    for t, name in ((vg, "gate values"), (mg, "gate masks"), (vu, "up values"), (mu, "up masks")):
        _dev(t, name)
    x2, squeeze = _x2(x)
    B, K = x2.shape
    R = mg.shape[0]
    if mg.shape != (R, K // 8) or mu.shape != mg.shape or vg.shape != (R, K // m * n) or vu.shape != vg.shape:
        raise ValueError("gate/up shapes do not match x and n:m")
    if vg.dtype != x.dtype or vu.dtype != x.dtype:
        raise ValueError("values must be in x's dtype")
    h = torch.empty((B, R), dtype=x.dtype, device=x.device) if out is None else _dev(out, "out")
    call("nm_spmv_swiglu", vg.data_ptr(), mg.data_ptr(), vu.data_ptr(), mu.data_ptr(), R, K, n, m,
         dtype_code(x.dtype), x2.data_ptr(), B, h.data_ptr(), stream_handle(stream))
    return h[0] if squeeze else h


def gemv_dense_swiglu(W_gate, W_up, x, out=None, stream=None):
    """Dense baseline of spmv_swiglu: h = SiLU(W_gate x) * (W_up x)."""
    _dev(W_gate, "W_gate"), _dev(W_up, "W_up")
    x2, squeeze = _x2(x)
    B, K = x2.shape
    R = W_gate.shape[0]
    if W_gate.shape != (R, K) or W_up.shape != (R, K) or W_gate.dtype != x.dtype or W_up.dtype != x.dtype:
        raise ValueError("W_gate/W_up must be [R][K] in x's dtype")
    h = torch.empty((B, R), dtype=x.dtype, device=x.device) if out is None else _dev(out, "out")
    call("nm_gemv_dense_swiglu", W_gate.data_ptr(), W_up.data_ptr(), R, K, dtype_code(x.dtype), x2.data_ptr(), B,
         h.data_ptr(), stream_handle(stream))
    return h[0] if squeeze else h


def calib_accumulate(X, decode=None, H=None, stream=None):
    """H += sum over decode rows t of X[t]^T X[t] (fp32 [K][K]).  X is [T][K]
    16-bit; decode is a bool/uint8 [T] tensor (nonzero = decode step) or None
    (all rows).  A new zeroed H is made when none is given."""
    _dev(X, "X")
    if X.dim() != 2:
        raise ValueError("X must be [T][K]")
    T, K = X.shape
    if H is None:
        H = torch.zeros((K, K), dtype=torch.float32, device=X.device)
    _dev(H, "H")
    if H.shape != (K, K) or H.dtype != torch.float32:
        raise ValueError("H must be float32 [K][K]")
    dp = None
    if decode is not None:
        _dev(decode, "decode")
        if decode.shape != (T,) or decode.dtype not in (torch.bool, torch.uint8):
            raise ValueError("decode must be a bool/uint8 [T] tensor")
        dp = decode.data_ptr()
    call("nm_calib_accumulate", X.data_ptr(), dp, T, K, dtype_code(X.dtype), H.data_ptr(), stream_handle(stream))
    return H


def calib_keep_mask(W, H, n=2, m=4, stream=None):
    """Keep-mask (uint8 [R][K], n ones per m-group) of the columns with the
    largest w^2 * H_jj; H is the [K][K] calibration Hessian or its diagonal [K]."""
    _dev(W, "W"), _dev(H, "H")
    R, K = W.shape
    if H.dtype != torch.float32:
        raise ValueError("H must be float32")
    if H.shape == (K, K):
        stride = K + 1
    elif H.shape == (K,):
        stride = 1
    else:
        raise ValueError("H must be [K][K] or [K]")
    keep = torch.empty((R, K), dtype=torch.uint8, device=W.device)
    call("nm_calib_keep_mask", W.data_ptr(), H.data_ptr(), stride, R, K, n, m, dtype_code(W.dtype), keep.data_ptr(),
         stream_handle(stream))
    return keep


class Hybrid:
    """A hybrid matrix: sparse rows packed (values, masks), dense rows as they
    are (W_dense), and the y rows of each (rows_sparse, rows_dense)."""

    def __init__(self, values, masks, W_dense, rows_sparse, rows_dense, R, K, n, m):
        self.values, self.masks, self.W_dense = values, masks, W_dense
        self.rows_sparse, self.rows_dense = rows_sparse, rows_dense
        self.R, self.K, self.n, self.m = R, K, n, m

    @property
    def n_dense(self):
        return self.rows_dense.shape[0]


def hybrid_row_loss(W, n=2, m=4, keep=None, H=None, stream=None):
    """Per-row pruning loss (float64 [R]): sum over pruned columns of w^2 * H_jj
    (H: [K][K] or its diagonal [K], float32; None for 1)."""
    _dev(W, "W")
    R, K = W.shape
    kp = None
    if keep is not None:
        _dev(keep, "keep")
        kp = keep.data_ptr()
    hp, hs = None, 0
    if H is not None:
        _dev(H, "H")
        if H.dtype != torch.float32:
            raise ValueError("H must be float32")
        hp, hs = H.data_ptr(), (K + 1 if H.shape == (K, K) else 1)
        if H.shape not in ((K, K), (K,)):
            raise ValueError("H must be [K][K] or [K]")
    loss = torch.empty(R, dtype=torch.float64, device=W.device)
    call("nm_hybrid_row_loss", W.data_ptr(), kp, hp, hs, R, K, n, m, dtype_code(W.dtype), loss.data_ptr(),
         stream_handle(stream))
    return loss


def hybrid_select_rows(loss, n_dense, stream=None):
    """uint8 [R] flags of the n_dense rows of largest loss."""
    _dev(loss, "loss")
    if loss.dtype != torch.float64 or loss.dim() != 1:
        raise ValueError("loss must be float64 [R]")
    flags = torch.empty(loss.shape[0], dtype=torch.uint8, device=loss.device)
    call("nm_hybrid_select_rows", loss.data_ptr(), loss.shape[0], n_dense, flags.data_ptr(), stream_handle(stream))
    return flags


def hybrid_pack(W, flags, n_dense=None, n=2, m=4, keep=None, stream=None):
    """Build a Hybrid from W and row flags (n_dense nonzero; counted on the
    host when not given)."""
    _dev(W, "W"), _dev(flags, "flags")
    R, K = W.shape
    if n_dense is None:
        n_dense = int(flags.count_nonzero().item())
    Rs = R - n_dense
    values = torch.empty((Rs, K // m * n), dtype=W.dtype, device=W.device)
    masks = torch.empty((Rs, K // 8), dtype=torch.uint8, device=W.device)
    W_dense = torch.empty((n_dense, K), dtype=W.dtype, device=W.device)
    rows_sparse = torch.empty(Rs, dtype=torch.int32, device=W.device)
    rows_dense = torch.empty(n_dense, dtype=torch.int32, device=W.device)
    kp = None
    if keep is not None:
        _dev(keep, "keep")
        kp = keep.data_ptr()
    call("nm_hybrid_pack", W.data_ptr(), kp, flags.data_ptr(), n_dense, R, K, n, m, dtype_code(W.dtype),
         values.data_ptr(), masks.data_ptr(), W_dense.data_ptr(), rows_sparse.data_ptr(), rows_dense.data_ptr(),
         stream_handle(stream))
    return Hybrid(values, masks, W_dense, rows_sparse, rows_dense, R, K, n, m)


def spmv_hybrid(hyb, x, out=None, stream=None):
    """y = W_hybrid x; x [K] or [B][K] -> [R] or [B][R]."""
    x2, squeeze = _x2(x)
    B, K = x2.shape
    if K != hyb.K:
        raise ValueError("x does not match the matrix")
    y = torch.empty((B, hyb.R), dtype=x.dtype, device=x.device) if out is None else _dev(out, "out")
    call("nm_spmv_hybrid", hyb.values.data_ptr(), hyb.masks.data_ptr(), hyb.rows_sparse.data_ptr(),
         hyb.W_dense.data_ptr(), hyb.rows_dense.data_ptr(), hyb.n_dense, hyb.R, K, hyb.n, hyb.m, dtype_code(x.dtype),
         x2.data_ptr(), B, y.data_ptr(), stream_handle(stream))
    return y[0] if squeeze else y
