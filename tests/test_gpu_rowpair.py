"""GPU parity of the row-slice kernel's row pairs (two rows a wave, sparse
formats, 3 and 4 vectors, rows of 4 or 5 chunks a lane): every output element
against the oracle, with ragged row counts (a last wave holding one row),
a partly filled last chunk slot, several matrices in one launch whose part
boundaries fall inside a pair, the gated launch (a pair is the gate and up
row of one output), integer-valued inputs that pin each sum exactly, and the
plain one-row-a-wave plan (NMSPMV_RPW=1, in a child process) giving the
same bits."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_matrix_vector_amd import inputs as I

pytestmark = pytest.mark.gpu

TD = {"fp16": torch.float16, "bf16": torch.bfloat16}
TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)


@pytest.fixture(scope="module")
def nm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_matrix_vector_amd as nm
    nm.lib()
    return nm


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def check_parts(nm, Rs, K, n, m, dt, B, seed, integer=False):
    """nm_spmv_multi over matrices of Rs rows sharing x, every element against the oracle."""
    tdt = TD[dt]
    if integer:
        Ws = [I.integer_valued(R, K, tdt, I.seed_of("pairW", R, K, n, m, dt, seed, i), scale=1 / 16)
              for i, R in enumerate(Rs)]
        x = I.integer_valued(B, K, tdt, I.seed_of("pairx", K, dt, B, seed), lo=-3, hi=3)
    else:
        Ws = [I.weight(R, K, tdt, I.seed_of("pairW", R, K, n, m, dt, seed, i)) for i, R in enumerate(Rs)]
        x = I.activation_normal(B, K, tdt, I.seed_of("pairx", K, dt, B, seed), outlier_frac=0.01)
    parts = [nm.pack(W.cuda(), None, n, m) for W in Ws]
    ys = nm.spmv_multi(parts, x.cuda(), n, m)
    torch.cuda.synchronize()
    worst = 0.0
    for W, (v, mk), y in zip(Ws, parts, ys):
        ov, om = oracle.pack(bits(W), None, n, m, dt)
        assert np.array_equal(bits(v), ov) and np.array_equal(mk.cpu().numpy(), om)
        yref, A = oracle.spmv(ov, om, K, n, m, dt, bits(x))
        if integer:
            # integer-valued inputs: every partial sum is exact in fp32, so y is the rounded exact sum
            assert np.array_equal(bits(y), oracle.round_to(yref, dt)), "integer-valued product not exact"
        ok, w, idx = oracle.check(bits(y), yref, A, dt)
        assert ok, f"outside tolerance: worst ratio {w:.3f} at {idx}"
        worst = max(worst, w)
    return worst


# Row counts with two blocks per CU at 16 rows a block (>= 8192 rows), odd
# counts (the last wave's second row past R), K with a partly filled last
# chunk slot (3600 columns: 225 sparse chunks, 4 a lane), both formats and
# dtypes, 3 and 4 vectors.
@pytest.mark.parametrize("R,K,n,m,dt,B", [
    (8192, 4096, 2, 4, "fp16", 3),
    (8193, 5120, 2, 4, "bf16", 3),
    (9001, 4096, 4, 8, "bf16", 4),
    (8193, 5120, 4, 8, "fp16", 3),
    (8705, 3600, 2, 4, "bf16", 4),
])
def test_rowpair_single(nm, R, K, n, m, dt, B):
    check_parts(nm, [R], K, n, m, dt, B, 1)


def test_rowpair_parts_boundaries_inside_pairs(nm):
    """Parts of odd row counts: pairs straddle the part boundaries."""
    check_parts(nm, [4097, 1023, 3001, 1], 4096, 2, 4, "fp16", 3, 2)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_rowpair_integer_exact(nm, n, m):
    check_parts(nm, [8201], 5120, n, m, "bf16", 4, 3, integer=True)


@pytest.mark.parametrize("dt,B", [("bf16", 3), ("fp16", 4)])
def test_rowpair_gated(nm, dt, B):
    import test_gpu_swiglu as W
    W.run_sparse(nm, 8192, 4096, 2, 4, dt, B, 4)


def _child():
    """Runs under NMSPMV_RPW=1: prints the one-row-a-wave outputs' bits."""
    import sparse_matrix_vector_amd as nm
    nm.lib()
    tdt = torch.bfloat16
    W = I.weight(8193, 5120, tdt, I.seed_of("pair_plain", 8193))
    x = I.activation_normal(4, 5120, tdt, I.seed_of("pair_plain_x"), outlier_frac=0.01)
    v, mk = nm.pack(W.cuda(), None, 2, 4)
    y = nm.spmv(v, mk, x.cuda(), 2, 4)
    torch.cuda.synchronize()
    np.save(sys.argv[1], bits(y))
    print(json.dumps({"ok": True}), flush=True)


def test_rowpair_against_one_row_a_wave(nm, tmp_path):
    """The row-pair plan gives the one-row-a-wave plan's bits: a lane forms
    each row's products and adds them in the same order in both, and the
    cross-lane reduction is the same."""
    tdt = torch.bfloat16
    W = I.weight(8193, 5120, tdt, I.seed_of("pair_plain", 8193))
    x = I.activation_normal(4, 5120, tdt, I.seed_of("pair_plain_x"), outlier_frac=0.01)
    v, mk = nm.pack(W.cuda(), None, 2, 4)
    y = nm.spmv(v, mk, x.cuda(), 2, 4)
    torch.cuda.synchronize()
    out = tmp_path / "plain.npy"
    env = {k: val for k, val in os.environ.items() if not k.startswith("NMSPMV_")}
    env.update({"NMSPMV_RPW": "1", "PYTHONPATH": os.pathsep.join([ROOT, TESTS])})
    proc = subprocess.run([sys.executable, "-c", "import sys, test_gpu_rowpair as t; t._child()", str(out)],
                          env=env, cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert proc.returncode == 0, (proc.stdout + proc.stderr)[-3000:]
    plain = np.load(out)
    assert np.array_equal(bits(y), plain), "row pairs and one row a wave differ"
