"""GPU parity of batched products (B = 4..32 activation vectors), which run
on the matrix cores: 2:4, 4:8 and dense, single and fused launches, the gated
epilogue, and the generic N:M path in batches of 8, against the oracle.  A
one-hot test checks the matrix-core operand and result layouts exactly."""
import numpy as np
import pytest
import torch

import oracle
from sparse_matrix_vector_amd import inputs as I

pytestmark = pytest.mark.gpu

TD = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def nm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_matrix_vector_amd as nm
    nm.lib()
    return nm


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def sample_rows(R, seed, k=16):
    g = np.random.default_rng(seed)
    return sorted({0, R // 2, R - 1} | set(g.choice(R, size=min(k, R), replace=False).tolist()))


def run_sparse(nm, R, K, n, m, dt, B, seed, rows=None, device_inputs=False):
    tdt = TD[dt]
    dev = "cuda" if device_inputs else "cpu"
    W = I.weight(R, K, tdt, I.seed_of("bW", R, K, n, m, dt, seed), device=dev)
    x = I.activation_normal(B, K, tdt, I.seed_of("bx", R, K, dt, B, seed), device=dev, outlier_frac=0.01)
    v, mk = nm.pack(W.cuda(), None, n, m)
    y = nm.spmv(v, mk, x.cuda(), n, m)
    torch.cuda.synchronize()
    assert y.shape == (B, R)
    rows = list(range(R)) if rows is None else rows
    ov, om = oracle.pack(bits(W[rows]), None, n, m, dt)
    assert np.array_equal(bits(v[rows]), ov) and np.array_equal(mk[rows].cpu().numpy(), om)
    yref, A = oracle.spmv(ov, om, K, n, m, dt, bits(x))
    ok, worst, idx = oracle.check(bits(y[:, rows]), yref, A, dt)
    assert ok, f"outside tolerance: worst {worst:.3f} at {idx}"


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("R,K", [(1, 16), (37, 1040), (130, 4096), (200, 16 * 600)])
@pytest.mark.parametrize("B", [4, 9, 16, 17, 32])
def test_spmv_batched(nm, dt, n, m, R, K, B):
    run_sparse(nm, R, K, n, m, dt, B, seed=1)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("R,B", [(4096, 24), (4112, 24), (4112, 32), (5000, 20)])
def test_spmv_batched_slice_rule(nm, n, m, R, B):
    """Above 16 vectors, rows too few for the LDS ring go to the staged
    kernel, which splits K in 2 slices, or keeps it whole from 24 vectors
    when the 16-row tiles outnumber the CUs (on 256 CUs: 4112 rows = 257
    tiles whole; 4096 rows at 24 and 5000 rows at 20 in 2 slices).  Every
    output is compared."""
    run_sparse(nm, R, 2048, n, m, "bf16", B, seed=7)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("B", [5, 16, 32])
def test_spmv_batched_integer_exact(nm, dt, n, m, B):
    """Exact sums: y must be the oracle's correctly rounded value bit for bit."""
    R, K = 77, 2048 + 64
    tdt = TD[dt]
    W = I.integer_valued(R, K, tdt, I.seed_of("bintW", dt, n, m), scale=1 / 16)
    x = I.integer_valued(B, K, tdt, I.seed_of("bintx", dt, n, m, B))
    ov, om = oracle.pack(bits(W), None, n, m, dt)
    yref, _ = oracle.spmv(ov, om, K, n, m, dt, bits(x))
    v, mk = nm.pack(W.cuda(), None, n, m)
    y = nm.spmv(v, mk, x.cuda(), n, m)
    assert np.array_equal(bits(y), oracle.round_to(yref, dt))


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_spmv_batched_one_hot_layout(nm, n, m):
    """x row b is the unit vector of column c_b: y[b] must be column c_b of the
    pruned matrix exactly.  16 different columns per launch cover every
    batch lane and, across rows, every result slot of the matrix-core tile."""
    R, K, B = 48, 256, 16
    W = I.weight(R, K, torch.float16, I.seed_of("ohW", n, m))
    v, mk = nm.pack(W.cuda(), None, n, m)
    ov, om = oracle.pack(bits(W), None, n, m, "fp16")
    wt = oracle.decode(oracle.expand(ov, om, K, n, m), "fp16")          # [R][K] pruned matrix
    for c0 in range(0, K, B):
        x = torch.zeros((B, K), dtype=torch.float16)
        for b in range(B):
            x[b, c0 + (b * 7) % B] = 1.0
        y = nm.spmv(v, mk, x.cuda(), n, m)
        got = oracle.decode(bits(y), "fp16")                            # [B][R]
        want = np.stack([wt[:, c0 + (b * 7) % B] for b in range(B)])
        assert np.array_equal(got, want), f"columns from {c0}"


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("R,K,B", [(45, 1000, 4), (130, 4096, 12), (16, 32768 + 512, 32)])
def test_gemv_dense_batched(nm, dt, R, K, B):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("bdW", R, K, dt))
    x = I.activation_normal(B, K, tdt, I.seed_of("bdx", R, K, dt, B), outlier_frac=0.01)
    yref, A = oracle.gemv(bits(W), dt, bits(x))
    y = nm.gemv_dense(W.cuda(), x.cuda())
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
@pytest.mark.parametrize("B", [6, 20])
def test_spmv_multi_batched(nm, n, m, B):
    """Fused parts whose boundaries fall inside 16-row tiles."""
    dt, tdt = "bf16", torch.bfloat16
    Rs, K = (40, 0, 77, 13), 2048 + 16 * 3
    x = I.activation_normal(B, K, tdt, I.seed_of("bmx", B, n, m))
    parts, ref = [], []
    for i, R in enumerate(Rs):
        W = I.weight(R, K, tdt, I.seed_of("bmW", i, R, n, m))
        ov, om = oracle.pack(bits(W), None, n, m, dt)
        ref.append(oracle.spmv(ov, om, K, n, m, dt, bits(x)))
        parts.append(nm.pack(W.cuda(), None, n, m))
    ys = nm.spmv_multi(parts, x.cuda(), n, m)
    for y, (yref, A), R in zip(ys, ref, Rs):
        assert y.shape == (B, R)
        ok, worst, idx = oracle.check(bits(y), yref, A, dt)
        assert ok, (R, worst, idx)


@pytest.mark.parametrize("n,m,K", [(1, 4, 24), (3, 8, 1000), (2, 4, 1032)])
def test_spmv_generic_batches_of_8(nm, n, m, K):
    """N:M patterns (or K % 16 != 0) outside the fast formats, B = 20: the
    generic kernel runs over x and y 8 rows at a time."""
    run_sparse(nm, 29, K, n, m, "fp16", 20, seed=3)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("B", [4, 16, 32])
def test_swiglu_batched(nm, dt, B):
    R, K, n, m = 300, 4096, 2, 4
    tdt = TD[dt]
    Wg = I.weight(R, K, tdt, I.seed_of("bgW", dt, B))
    Wu = I.weight(R, K, tdt, I.seed_of("buW", dt, B))
    x = I.activation_normal(B, K, tdt, I.seed_of("bgx", dt, B), outlier_frac=0.01)
    g, u = nm.pack(Wg.cuda(), None, n, m), nm.pack(Wu.cuda(), None, n, m)
    h = nm.spmv_swiglu(g, u, x.cuda(), n, m)
    hd = nm.gemv_dense_swiglu(Wg.cuda(), Wu.cuda(), x.cuda())
    gv, gm = oracle.pack(bits(Wg), None, n, m, dt)
    uv, um = oracle.pack(bits(Wu), None, n, m, dt)
    gref, Ag = oracle.spmv(gv, gm, K, n, m, dt, bits(x))
    uref, Au = oracle.spmv(uv, um, K, n, m, dt, bits(x))
    ok, worst, idx = oracle.check_swiglu(bits(h), gref, uref, Ag, Au, dt)
    assert ok, ("sparse", worst, idx)
    gdr, Agd = oracle.gemv(bits(Wg), dt, bits(x))
    udr, Aud = oracle.gemv(bits(Wu), dt, bits(x))
    ok, worst, idx = oracle.check_swiglu(bits(hd), gdr, udr, Agd, Aud, dt)
    assert ok, ("dense", worst, idx)


@pytest.mark.parametrize("name,B", [("gate", 16), ("down", 32)])
def test_qwen3_32b_batched_full_size(nm, name, B):
    """Qwen3-32B MLP shapes (2:4 bf16) at B = 16 and 32, sampled rows."""
    R, K = I.QWEN3_32B_MLP[name]
    run_sparse(nm, R, K, 2, 4, "bf16", B, seed=4, rows=sample_rows(R, 5), device_inputs=True)
