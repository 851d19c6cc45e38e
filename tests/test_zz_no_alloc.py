"""The allocation-free entry point (nm_spmv_multi_noalloc) against the
workspace call it mirrors (nm_spmv_multi_ws), through the C ABI: two calls in
a row on the K-split plan's shapes, the second smaller, each compared with
the workspace call bit for bit and with the oracle element by element."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_matrix_vector_amd import inputs as I

pytestmark = pytest.mark.gpu

P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def run_pair(nm, lib, ws, R, K, B, seed):
    W = I.weight(R, K, torch.bfloat16, I.seed_of("noallocW", R, K, seed))
    x = I.activation_normal(B, K, torch.bfloat16, I.seed_of("noallocx", R, K, B, seed), outlier_frac=0.01)
    values, masks = nm.pack(W.cuda(), None, 2, 4)
    xc = x.cuda()
    y_na = torch.empty((B, R), dtype=torch.bfloat16, device="cuda")
    y_ws = torch.empty((B, R), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    common = (I32(1), (P * 1)(values.data_ptr()), (P * 1)(masks.data_ptr()), (I64 * 1)(R), I64(K), I32(2), I32(4),
              I32(1), P(xc.data_ptr()), I32(B))
    assert lib.nm_spmv_multi_noalloc(*common, (P * 1)(y_na.data_ptr()), P(stream)) == 0
    assert lib.nm_spmv_multi_ws(*common, (P * 1)(y_ws.data_ptr()), P(ws.data_ptr()), I64(ws.numel()), P(stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws), "allocation-free and workspace calls differ"
    ov, om = oracle.pack(bits(W), None, 2, 4, "bf16")
    yref, A = oracle.spmv(ov, om, K, 2, 4, "bf16", bits(x))
    ok, worst, idx = oracle.check(bits(y_na), yref, A, "bf16")
    assert ok, f"outside tolerance: worst ratio {worst:.3f} at {idx}"


def test_noalloc_matches_workspace_call_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_matrix_vector_amd as nm
    lib = nm.lib()
    ws = nm.workspace()
    run_pair(nm, lib, ws, 320, 16384, 8, 1)          # K-split plan: 160 tile groups
    run_pair(nm, lib, ws, 97, 8192, 8, 2)            # smaller: fewer groups, other splits, a ragged tile
