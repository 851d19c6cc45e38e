"""GPU parity under every launch-shape override (the NMSPMV_* tuning
variables), each in a child process of its own, since the library reads them
once per process.  Each child runs a fixed set of products -- single vectors
on long and short rows, small batches, the matrix-core batches, the gated
call, several matrices in one launch, the hybrid product -- through the C ABI
and checks every output element against the oracle with the suites' own
checkers.  Overrides change only how the work is laid out, never the result's
tolerance."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)

# (R, K, n, m, dtype, B): long rows at the single-vector sizes where the
# overrides change the plan (one wave per row up to 16 chunks a lane, slices,
# the stream kernel), short rows, batches on both sides of the matrix-core
# switch, and ragged row counts.
CASES = [
    (300, 14336, 2, 4, "fp16", 1),     # 896 chunks a row
    (97, 16384, 2, 4, "bf16", 1),      # 1024 chunks: 16 a lane on one wave
    (130, 9216, 4, 8, "bf16", 1),      # 576 chunks: 9 a lane
    (200, 12288, 2, 4, "fp16", 1),     # 768 chunks: 12 a lane
    (515, 4096, 2, 4, "fp16", 1),
    (1030, 1040, 4, 8, "bf16", 3),
    (257, 14336, 2, 4, "bf16", 2),
    (300, 5120, 2, 4, "bf16", 8),
    (100, 8192, 4, 8, "fp16", 16),
    (70, 2080, 2, 4, "fp16", 32),
    (8193, 4096, 2, 4, "bf16", 3),     # row pairs (two rows a wave) by default
]
# run only under the override that changes their plan
CASES_FOR = {"NMSPMV_RPW": [(8192, 5120, 2, 4, "fp16", 2), (8201, 4096, 4, 8, "bf16", 1)]}   # row pairs from 1 vector

SETTINGS = [
    {"NMSPMV_MAX_CPL": "16"},
    {"NMSPMV_MAX_CPL": "10"},
    {"NMSPMV_MAX_CPL": "14", "NMSPMV_ROWS_PER_BLOCK": "4"},
    {"NMSPMV_KERNEL": "3"},
    {"NMSPMV_KERNEL": "3", "NMSPMV_THREADS": "256", "NMSPMV_TILE_BYTES": "4096"},
    {"NMSPMV_KERNEL": "1", "NMSPMV_SLICES": "16"},
    {"NMSPMV_ROWS_PER_BLOCK": "3"},
    {"NMSPMV_XDMA": "1"},
    {"NMSPMV_XFIRST": "0"},
    {"NMSPMV_XFIRST": "1"},
    {"NMSPMV_BLOCKS_PER_CU": "2"},
    {"NMSPMV_KERNEL": "5"},
    {"NMSPMV_KERNEL": "6"},
    {"NMSPMV_MFMA_MIN_B": "2"},
    {"NMSPMV_MFMA_SLICES": "3"},
    {"NMSPMV_RING_TILES": "2"},
    {"NMSPMV_RING_SHARE": "8"},
    {"NMSPMV_HYBRID_SPLIT": "1"},
    {"NMSPMV_SPLITK": "2"},
    {"NMSPMV_SPLITK": "2", "NMSPMV_SPLITK_KS": "3"},
    {"NMSPMV_SPLITK": "1"},
    {"NMSPMV_RPW": "1"},
    {"NMSPMV_RPW": "2"},
]


def child():
    """Runs in the child process: every case under the inherited overrides."""
    import numpy as np
    import torch

    import oracle
    import sparse_matrix_vector_amd as nm
    import test_gpu_hybrid as H
    import test_gpu_parity as G
    import test_gpu_swiglu as W
    from sparse_matrix_vector_amd import inputs as I
    nm.lib()
    worst = 0.0
    cases = list(CASES)
    for var, extra in CASES_FOR.items():
        if os.environ.get(var) == "2":
            cases += extra
    for seed, (R, K, n, m, dt, B) in enumerate(cases):
        print(json.dumps({"case": [R, K, n, m, dt, B]}), flush=True)
        worst = max(worst, G.run_case(nm, R, K, n, m, dt, B, 700 + seed))
    print(json.dumps({"case": "swiglu"}), flush=True)
    worst = max(worst, W.run_sparse(nm, 130, 9216, 2, 4, "bf16", 1, 7))
    worst = max(worst, W.run_sparse(nm, 257, 4096, 4, 8, "fp16", 8, 8))
    # several matrices in one launch (q+k+v-like), long rows
    print(json.dumps({"case": "multi"}), flush=True)
    tdt = G.TD["fp16"]
    K = 14336
    Ws = [I.weight(R, K, tdt, I.seed_of("knob_multi", R, K)) for R in (96, 33, 160)]
    x = I.activation_normal(1, K, tdt, I.seed_of("knob_multi_x", K), outlier_frac=0.01)
    packed = [nm.pack(W.cuda(), None, 2, 4) for W in Ws]
    ys = nm.spmv_multi(packed, x.cuda(), 2, 4)
    torch.cuda.synchronize()
    for W, y in zip(Ws, ys):
        ov, om = oracle.pack(G.bits(W), None, 2, 4, "fp16")
        yref, A = oracle.spmv(ov, om, K, 2, 4, "fp16", G.bits(x))
        ok, w, idx = oracle.check(G.bits(y), yref, A, "fp16")
        assert ok, ("multi", w, idx)
        worst = max(worst, w)
    # with a K-split workspace: batched, few rows (and, with the plan forced, any ring shape)
    print(json.dumps({"case": "workspace"}), flush=True)
    ws = nm.workspace()
    for R, K, B in ((160, 16384, 8), (1030, 4096, 16), (70, 2080, 32)):
        Wk = I.weight(R, K, tdt, I.seed_of("knob_ws", R, K))
        xk = I.activation_normal(B, K, tdt, I.seed_of("knob_ws_x", K, B), outlier_frac=0.01)
        yk = nm.spmv_multi([nm.pack(Wk.cuda(), None, 2, 4)], xk.cuda(), 2, 4, ws=ws)[0]
        ov, om = oracle.pack(G.bits(Wk), None, 2, 4, "fp16")
        yref, A = oracle.spmv(ov, om, K, 2, 4, "fp16", G.bits(xk))
        ok, w, idx = oracle.check(G.bits(yk), yref, A, "fp16")
        assert ok, ("workspace", R, K, B, w, idx)
        worst = max(worst, w)
    # hybrid rows, at one vector (one launch) and at three
    print(json.dumps({"case": "hybrid"}), flush=True)
    for B in (1, 3):
        R, K = 600, 8192
        W = I.weight(R, K, tdt, I.seed_of("knob_hyb", R, K))
        xh = I.activation_normal(B, K, tdt, I.seed_of("knob_hyb_x", K, B), outlier_frac=0.01)
        nd = 60
        flags = nm.hybrid_select_rows(nm.hybrid_row_loss(W.cuda(), 2, 4), nd)
        hyb = nm.hybrid_pack(W.cuda(), flags, nd, 2, 4)
        y = nm.spmv_hybrid(hyb, xh.cuda())
        f = flags.cpu().numpy().astype(bool)
        yref, A = oracle.hybrid_spmv(G.bits(W), f, 2, 4, "fp16", G.bits(xh))
        ok, w, idx = oracle.check(G.bits(y), yref, A, "fp16")
        assert ok, ("hybrid", B, w, idx)
        worst = max(worst, w)
    assert np.isfinite(worst)
    print(json.dumps({"ok": True, "worst_ratio": worst}), flush=True)


@pytest.mark.parametrize("setting", SETTINGS, ids=lambda s: ",".join(f"{k[7:]}={v}" for k, v in s.items()))
def test_parity_under_override(setting):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = {k: v for k, v in os.environ.items() if not k.startswith("NMSPMV_")}
    env.update(setting)
    env["PYTHONPATH"] = os.pathsep.join([ROOT, TESTS])
    proc = subprocess.run([sys.executable, "-c", "import test_gpu_knobs as t; t.child()"], env=env, cwd=ROOT,
                          capture_output=True, text=True, timeout=240)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0, out[-3000:]
    assert '"ok": true' in proc.stdout
