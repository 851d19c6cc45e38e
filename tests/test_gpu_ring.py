"""GPU parity of the LDS-ring matrix-core kernel's configurations through the
C ABI, against the oracle: one 16-row tile per wave (5 to 8 vectors), two (9
to 16, and above 16 with two batch tiles), x shared by the waves of a block
when a tile keeps one K-slice; odd batch sizes
(x rows are staged in pairs, the last one repeated), K with a partial last
stage, row counts that end inside a wave's tiles, fused launches whose part
boundaries fall inside a wave's rows, and the gated epilogue."""
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


def sparse_case(nm, W, x, n, m, dt, rows=None):
    v, mk = nm.pack(W if W.is_cuda else W.cuda(), None, n, m)
    y = nm.spmv(v, mk, x.cuda(), n, m)
    rows = list(range(W.shape[0])) if rows is None else rows
    ov, om = oracle.pack(bits(W[rows]), None, n, m, dt)
    yref, A = oracle.spmv(ov, om, W.shape[1], n, m, dt, bits(x))
    ok, worst, idx = oracle.check(bits(y[:, rows]), yref, A, dt)
    assert ok, f"outside tolerance: worst {worst:.3f} at {idx}"


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("B", [5, 7, 8, 9, 13, 16])
@pytest.mark.parametrize("R,K", [(37, 1056), (200, 4128), (1000, 8192)])
def test_ring_sparse(nm, dt, n, m, B, R, K):
    """K = 1056 and 4128 end in a partial stage (66 and 258 chunks of 16)."""
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("rgW", R, K, n, m, dt))
    x = I.activation_normal(B, K, tdt, I.seed_of("rgx", R, K, dt, B), outlier_frac=0.01)
    sparse_case(nm, W, x, n, m, dt)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("B", [7, 13])
def test_ring_sparse_integer_exact(nm, dt, n, m, B):
    """Exact sums: one and two tiles per wave bit for bit."""
    R, K = 77, 2080
    tdt = TD[dt]
    W = I.integer_valued(R, K, tdt, I.seed_of("rgiW", dt, n, m), scale=1 / 16)
    x = I.integer_valued(B, K, tdt, I.seed_of("rgix", dt, n, m, B))
    ov, om = oracle.pack(bits(W), None, n, m, dt)
    yref, _ = oracle.spmv(ov, om, K, n, m, dt, bits(x))
    v, mk = nm.pack(W.cuda(), None, n, m)
    y = nm.spmv(v, mk, x.cuda(), n, m)
    assert np.array_equal(bits(y), oracle.round_to(yref, dt))


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("B", [17, 25, 32])
def test_ring_sparse_above_16(nm, dt, n, m, B):
    """Above 16 vectors (two batch tiles) on a matrix with one 64-row block
    per CU and 40 rows more: two waves of two tiles share x, and the last
    block's tiles end inside the matrix; sampled rows, including the last
    40."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    R, K = 64 * cus + 40, 1056
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("rg4W", n, m, dt), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("rg4x", dt, B), device="cuda", outlier_frac=0.01)
    g = np.random.default_rng(I.seed_of("rg4r", B))
    rows = sorted(set(g.choice(R, size=40, replace=False).tolist()) | set(range(R - 40, R)) | {0, 63, 64})
    sparse_case(nm, W, x, n, m, dt, rows=rows)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("B", [5, 12, 17, 24, 32])
@pytest.mark.parametrize("R,K", [(70, 1000), (300, 4104)])
def test_ring_dense(nm, dt, B, R, K):
    """Dense rows: chunks of 8 columns, so K = 1000 and 4104 end in a partial
    stage; above 16 vectors two batch tiles share each weight operand."""
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("rgdW", R, K, dt))
    x = I.activation_normal(B, K, tdt, I.seed_of("rgdx", R, K, dt, B), outlier_frac=0.01)
    y = nm.gemv_dense(W.cuda(), x.cuda())
    yref, A = oracle.gemv(bits(W), dt, bits(x))
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("B", [6, 12])
def test_ring_multi_part(nm, n, m, B):
    """Fused parts of 40, 0, 77 and 13 rows: boundaries inside 16- and
    32-row wave tiles."""
    dt, tdt = "fp16", torch.float16
    Rs, K = (40, 0, 77, 13), 2048
    x = I.activation_normal(B, K, tdt, I.seed_of("rgmx", B, n, m))
    parts, ref = [], []
    for i, R in enumerate(Rs):
        W = I.weight(R, K, tdt, I.seed_of("rgmW", i, R, n, m))
        ov, om = oracle.pack(bits(W), None, n, m, dt)
        ref.append(oracle.spmv(ov, om, K, n, m, dt, bits(x)))
        parts.append(nm.pack(W.cuda(), None, n, m))
    ys = nm.spmv_multi(parts, x.cuda(), n, m)
    for y, (yref, A), R in zip(ys, ref, Rs):
        assert y.shape == (B, R)
        ok, worst, idx = oracle.check(bits(y), yref, A, dt)
        assert ok, (R, worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("B", [6, 12])
def test_ring_swiglu(nm, dt, B):
    """Gated epilogue with one and two tiles per wave, sparse and dense."""
    R, K, n, m = 300, 2080, 2, 4
    tdt = TD[dt]
    Wg = I.weight(R, K, tdt, I.seed_of("rggW", dt, B))
    Wu = I.weight(R, K, tdt, I.seed_of("rguW", dt, B))
    x = I.activation_normal(B, K, tdt, I.seed_of("rggx", dt, B), outlier_frac=0.01)
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


def _large_R(extra):
    """Enough 16-row tiles that a launch with one K-slice fills every CU with
    blocks of four waves sharing x, plus `extra` rows (a partial last block)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 64 * cus + extra


def _sample(R, seed, k=48):
    g = np.random.default_rng(seed)
    return sorted(set(g.choice(R, size=k, replace=False).tolist()) | set(range(R - 40, R)) | {0, 15, 16, 63, 64})


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("B", [5, 8, 9, 16])
def test_ring_shared_x(nm, dt, n, m, B):
    """Blocks whose waves share one staged x: four waves of one tile (up to 8
    vectors) or two of two tiles (9 to 16); K = 1056 ends in a partial stage,
    R in the middle of a block."""
    R, K = _large_R(40), 1056
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("rgsW", n, m, dt), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("rgsx", dt, B), device="cuda", outlier_frac=0.01)
    sparse_case(nm, W, x, n, m, dt, rows=_sample(R, I.seed_of("rgsr", B)))


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("B", [4, 8, 12, 20, 32])
def test_ring_shared_x_dense(nm, dt, B):
    """K = 504: 63 chunks of 8 columns, under 8 stages, so one K-slice and
    blocks that share x (above 16 vectors with two batch tiles)."""
    R, K = _large_R(24), 504
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("rgsdW", dt), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("rgsdx", dt, B), device="cuda", outlier_frac=0.01)
    y = nm.gemv_dense(W, x)
    rows = _sample(R, I.seed_of("rgsdr", B))
    yref, A = oracle.gemv(bits(W[rows]), dt, bits(x))
    ok, worst, idx = oracle.check(bits(y[:, rows]), yref, A, dt)
    assert ok, (worst, idx)


@pytest.mark.parametrize("B", [6, 12])
def test_ring_shared_x_swiglu_and_parts(nm, B):
    """The gated epilogue (launch rows interleave gate and up) and a fused
    launch of three parts, both on blocks that share x."""
    dt, tdt, n, m = "bf16", torch.bfloat16, 2, 4
    Rh, K = _large_R(8) // 2, 1056                 # 5 stages: one K-slice
    Wg = I.weight(Rh, K, tdt, I.seed_of("rgsgW", B), device="cuda")
    Wu = I.weight(Rh, K, tdt, I.seed_of("rgsuW", B), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("rgsgx", B), device="cuda", outlier_frac=0.01)
    g, u = nm.pack(Wg, None, n, m), nm.pack(Wu, None, n, m)
    h = nm.spmv_swiglu(g, u, x, n, m)
    rows = _sample(Rh, I.seed_of("rgsgr", B), k=32)
    gv, gm = oracle.pack(bits(Wg[rows]), None, n, m, dt)
    uv, um = oracle.pack(bits(Wu[rows]), None, n, m, dt)
    gref, Ag = oracle.spmv(gv, gm, K, n, m, dt, bits(x))
    uref, Au = oracle.spmv(uv, um, K, n, m, dt, bits(x))
    ok, worst, idx = oracle.check_swiglu(bits(h[:, rows]), gref, uref, Ag, Au, dt)
    assert ok, ("swiglu", worst, idx)
    # three parts: the first two end inside blocks of 64 rows
    Rs = (Rh + 7, 33, Rh - 1)
    Ws = [I.weight(R, K, tdt, I.seed_of("rgspW", i, B), device="cuda") for i, R in enumerate(Rs)]
    ys = nm.spmv_multi([nm.pack(Wp, None, n, m) for Wp in Ws], x, n, m)
    for i, (Wp, y, R) in enumerate(zip(Ws, ys, Rs)):
        rr = sorted(set(_sample(R, I.seed_of("rgspr", i, B), k=16)) | {R - 1}) if R > 64 else list(range(R))
        ov, om = oracle.pack(bits(Wp[rr]), None, n, m, dt)
        yref, A = oracle.spmv(ov, om, K, n, m, dt, bits(x))
        ok, worst, idx = oracle.check(bits(y[:, rr]), yref, A, dt)
        assert ok, ("part", i, worst, idx)


def _round_R(extra):
    """More 16-row tiles than four-wave blocks fit on the CUs at once (12 per
    CU plus 200), so the share is widened to fit every block in one round;
    `extra` rows end in a partial tile, and the last block is partial too."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 16 * (12 * cus + 200) + extra


@pytest.mark.parametrize("dt,n,m,B", [("fp16", 2, 4, 8), ("bf16", 4, 8, 5), ("bf16", 2, 4, 6), ("fp16", 4, 8, 7)])
def test_ring_shared_x_one_round(nm, dt, n, m, B):
    """Blocks of more than four waves sharing x (the share chosen so that no
    second round of blocks is left); sampled rows, the last 40 included."""
    R, K = _round_R(9), 1056
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("rg1W", n, m, dt), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("rg1x", dt, B), device="cuda", outlier_frac=0.01)
    sparse_case(nm, W, x, n, m, dt, rows=_sample(R, I.seed_of("rg1r", B), k=64))


def test_ring_shared_x_one_round_swiglu(nm):
    """The gated epilogue on the widened share (gate and up rows interleaved)."""
    dt, tdt, n, m, B = "bf16", torch.bfloat16, 2, 4, 8
    Rh, K = _round_R(5) // 2, 1056
    Wg = I.weight(Rh, K, tdt, I.seed_of("rg1gW"), device="cuda")
    Wu = I.weight(Rh, K, tdt, I.seed_of("rg1uW"), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("rg1gx"), device="cuda", outlier_frac=0.01)
    h = nm.spmv_swiglu(nm.pack(Wg, None, n, m), nm.pack(Wu, None, n, m), x, n, m)
    rows = _sample(Rh, I.seed_of("rg1gr"), k=48)
    gv, gm = oracle.pack(bits(Wg[rows]), None, n, m, dt)
    uv, um = oracle.pack(bits(Wu[rows]), None, n, m, dt)
    gref, Ag = oracle.spmv(gv, gm, K, n, m, dt, bits(x))
    uref, Au = oracle.spmv(uv, um, K, n, m, dt, bits(x))
    ok, worst, idx = oracle.check_swiglu(bits(h[:, rows]), gref, uref, Ag, Au, dt)
    assert ok, ("swiglu", worst, idx)
