"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Packing must be byte-identical; products must meet
|y_gpu - y_ref| <= 2e-3 * sum|w*x| + 1 ulp of the output format per element;
one-hot and integer-valued inputs must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from sparse_matrix_vector_amd import inputs as I

pytestmark = pytest.mark.gpu

TD = {"fp16": torch.float16, "bf16": torch.bfloat16}
NM_ALL = [(n, m) for m in (4, 8) for n in range(1, m)]


@pytest.fixture(scope="module")
def nm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_matrix_vector_amd as nm
    nm.lib()
    return nm


def bits(t):
    """torch 16-bit tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def gpu(t):
    return t.to("cuda")


def run_case(nm, R, K, n, m, dt, B, seed, keep=False, ties=False, xkind="normal"):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("W", R, K, n, m, dt, seed))
    if ties:
        W = (torch.round(W.float() / 0.01) * 0.01).to(tdt)
    kp = I.keep_mask(R, K, n, m, I.seed_of("keep", R, K, n, m, seed)) if keep else None
    if xkind == "laplace":
        x = I.activation_laplace(B, K, tdt, I.seed_of("x", R, K, dt, B, seed))
    else:
        x = I.activation_normal(B, K, tdt, I.seed_of("x", R, K, dt, B, seed), outlier_frac=0.01)
    # oracle side
    ov, om = oracle.pack(bits(W), None if kp is None else kp.numpy(), n, m, dt)
    yref, A = oracle.spmv(ov, om, K, n, m, dt, bits(x))
    # GPU side
    gv, gm = nm.pack(gpu(W), None if kp is None else gpu(kp), n, m)
    y = nm.spmv(gv, gm, gpu(x), n, m)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gv), ov), "packed values differ"
    assert np.array_equal(gm.cpu().numpy(), om), "masks differ"
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, f"tolerance exceeded: worst ratio {worst:.3f} at {idx}"
    return worst


# ---- pack ------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", NM_ALL)
@pytest.mark.parametrize("R,K", [(1, 8), (7, 72), (33, 1040)])
@pytest.mark.parametrize("keep", [False, True])
def test_pack_bitexact(nm, dt, n, m, R, K, keep):
    if K % m:
        pytest.skip("K must be a multiple of m")
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("packW", R, K, n, m, dt))
    W = (torch.round(W.float() / 0.005) * 0.005).to(tdt)        # many equal magnitudes -> ties
    W[0, : min(K, 8)] = -W[0, : min(K, 8)]
    kp = I.keep_mask(R, K, n, m, I.seed_of("packK", R, K, n, m)) if keep else None
    ov, om = oracle.pack(bits(W), None if kp is None else kp.numpy(), n, m, dt)
    gv, gm = nm.pack(gpu(W), None if kp is None else gpu(kp), n, m)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gv), ov)
    assert np.array_equal(gm.cpu().numpy(), om)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_pack_special_words(nm, dt):
    """Signed zeros, subnormals and infinities in top-N mode: the GPU's
    unsigned compare of (bits & 0x7FFF) must pick what the oracle's exact |w|
    picks."""
    rng = np.random.default_rng(7)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0002, 0x03FF, 0x0400, 0x7BFF, 0xFBFF,
                         0x7C00, 0xFC00, 0x3C00, 0xBC00] if dt == "fp16" else
                        [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                         0x3F80, 0xBF80], np.uint16)
    Wb = rng.choice(specials, size=(16, 256)).astype(np.uint16)
    W = torch.from_numpy(Wb.view(np.int16)).view(TD[dt])
    for n, m in NM_ALL:
        ov, om = oracle.pack(Wb, None, n, m, dt)
        gv, gm = nm.pack(gpu(W), None, n, m)
        torch.cuda.synchronize()
        assert np.array_equal(bits(gv), ov), (n, m)
        assert np.array_equal(gm.cpu().numpy(), om), (n, m)


def test_pack_config1_seed0(nm):
    """1024 x 1024 fp16 ~ N(0, 0.02), top-2 of 4, lowest index wins ties, seed 0."""
    W = I.weight(1024, 1024, torch.float16, 0)
    ov, om = oracle.pack(bits(W), None, 2, 4, "fp16")
    gv, gm = nm.pack(gpu(W), None, 2, 4)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gv), ov) and np.array_equal(gm.cpu().numpy(), om)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_pack_errors_leave_outputs_untouched(nm, dt):
    from sparse_matrix_vector_amd import _lib as L
    R, K = 8, 64
    W = gpu(I.weight(R, K, TD[dt], 3))
    keep = I.keep_mask(R, K, 2, 4, 3)
    keep[5, 9] ^= 1                                              # one group now has 1 or 3 kept
    vals = torch.full((R, K // 2), 1234, dtype=torch.int16, device="cuda").view(TD[dt])
    masks = torch.full((R, K // 8), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    st = L.lib().nm_pack(W.data_ptr(), gpu(keep).data_ptr(), R, K, 2, 4, 0 if dt == "fp16" else 1,
                         vals.data_ptr(), masks.data_ptr(), s)
    assert st == L.NM_ERR_BAD_MASK
    Wn = W.clone()
    Wn.view(torch.int16)[3, 17] = 0x7E00 if dt == "fp16" else 0x7FC0
    st = L.lib().nm_pack(Wn.data_ptr(), None, R, K, 2, 4, 0 if dt == "fp16" else 1, vals.data_ptr(),
                         masks.data_ptr(), s)
    assert st == L.NM_ERR_NONFINITE
    torch.cuda.synchronize()
    assert torch.all(vals.view(torch.int16) == 1234) and torch.all(masks == 0xA5)
    # keep-mask mode copies a NaN word verbatim
    good = I.keep_mask(R, K, 2, 4, 4)
    good[3, 16:20] = torch.tensor([0, 1, 1, 0], dtype=torch.uint8)
    gv, gm = nm.pack(Wn, gpu(good), 2, 4)
    ov, om = oracle.pack(bits(Wn), good.numpy(), 2, 4, dt)
    assert np.array_equal(bits(gv), ov) and np.array_equal(gm.cpu().numpy(), om)


# ---- sparse product ----------------------------------------------------------

@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("R,K", [(1, 16), (37, 1040), (130, 4096), (64, 1024 * 3 + 16 * 7)])
@pytest.mark.parametrize("B", [1, 2, 8])
def test_spmv_half_density(nm, dt, n, m, R, K, B):
    run_case(nm, R, K, n, m, dt, B, seed=11)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", NM_ALL)
@pytest.mark.parametrize("R,K,B", [(5, 24, 1), (29, 1000, 3), (40, 2056, 8)])
def test_spmv_any_nm(nm, dt, n, m, R, K, B):
    if K % m:
        K += m - K % m
    if K % 8:
        K += 8 - K % 8
    run_case(nm, R, K, n, m, dt, B, seed=12, keep=(n + m) % 2 == 0)


@pytest.mark.parametrize("B", [1, 3, 4, 5, 6, 7, 8])
def test_spmv_multi_tile(nm, B):
    """B * K * 2 bytes beyond one LDS tile: x is staged in several tiles."""
    run_case(nm, 48, 32768 + 1024, 2, 4, "bf16", B, seed=13, xkind="laplace")


def test_spmv_config1(nm):
    """1024 x 1024, 2:4, fp16, x ~ N(0,1), batch 1, seed 0."""
    W = I.weight(1024, 1024, torch.float16, 0)
    x = I.activation_normal(1, 1024, torch.float16, I.seed_of("x", 0))
    ov, om = oracle.pack(bits(W), None, 2, 4, "fp16")
    yref, A = oracle.spmv(ov, om, 1024, 2, 4, "fp16", bits(x))
    gv, gm = nm.pack(gpu(W), None, 2, 4)
    y = nm.spmv(gv, gm, gpu(x), 2, 4)
    ok, worst, idx = oracle.check(bits(y), yref, A, "fp16")
    assert ok, (worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (3, 8)])
def test_spmv_one_hot_bitexact(nm, dt, n, m):
    """x = e_j: y = column j of the pruned matrix exactly, subnormal weights
    included (the tolerance alone could not see one misplaced term)."""
    R, K = 96, 1024 if n * 2 == m else 512
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("onehot", dt, n, m))
    Wi = W.view(torch.int16)
    Wi[:, ::7] = torch.randint(1, 0x7F, Wi[:, ::7].shape, dtype=torch.int16)   # positive subnormals
    Wi[1::2, ::11] |= -0x8000                                                  # and negative ones
    ov, om = oracle.pack(bits(W), None, n, m, dt)
    wt = oracle.decode(oracle.expand(ov, om, K, n, m), dt)                      # [R][K]
    gv, gm = nm.pack(gpu(W), None, n, m)
    one = torch.ones((), dtype=tdt)
    for j0 in range(0, K, 8):
        x = torch.zeros((8, K), dtype=tdt)
        x[torch.arange(8), torch.arange(j0, j0 + 8)] = one
        y = nm.spmv(gv, gm, gpu(x), n, m)
        got = oracle.decode(bits(y), dt)                                        # [8][R]
        assert np.array_equal(got, wt[:, j0:j0 + 8].T), f"columns {j0}..{j0 + 7}"


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
@pytest.mark.parametrize("B", [1, 8])
def test_spmv_integer_exact(nm, dt, n, m, B):
    """w in {-8..8}/16, x in {-8..8}: every fp32 partial sum is exact, so y must
    be the oracle's correctly rounded value bit for bit in any order."""
    R, K = 77, 2048 + 64
    tdt = TD[dt]
    W = I.integer_valued(R, K, tdt, I.seed_of("intW", dt, n, m), scale=1 / 16)
    x = I.integer_valued(B, K, tdt, I.seed_of("intx", dt, n, m, B))
    ov, om = oracle.pack(bits(W), None, n, m, dt)
    yref, _ = oracle.spmv(ov, om, K, n, m, dt, bits(x))
    gv, gm = nm.pack(gpu(W), None, n, m)
    y = nm.spmv(gv, gm, gpu(x), n, m)
    assert np.array_equal(bits(y), oracle.round_to(yref, dt))


def test_spmv_empty_and_degenerate(nm):
    tdt = torch.float16
    # K == 0: every output is the empty sum
    v = torch.empty((5, 0), dtype=tdt, device="cuda")
    mk = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    x = torch.empty((3, 0), dtype=tdt, device="cuda")
    y = torch.full((3, 5), 7, dtype=tdt, device="cuda")
    nm.spmv(v, mk, x, 2, 4, out=y)
    assert torch.all(y == 0)
    # R == 0
    v = torch.empty((0, 32), dtype=tdt, device="cuda")
    mk = torch.empty((0, 8), dtype=torch.uint8, device="cuda")
    y = nm.spmv(v, mk, torch.ones((2, 64), dtype=tdt, device="cuda"), 2, 4)
    assert y.shape == (2, 0)
    # all-zero weights: kept zeros give +0
    W = torch.zeros((3, 64), dtype=tdt, device="cuda")
    gv, gm = nm.pack(W, None, 2, 4)
    assert torch.all(gm.cpu() == 0x33)
    y = nm.spmv(gv, gm, torch.ones((1, 64), dtype=tdt, device="cuda"), 2, 4)
    assert torch.all(y == 0)


def test_spmv_deterministic(nm):
    W = gpu(I.weight(512, 4096, torch.bfloat16, 21))
    x = gpu(I.activation_laplace(4, 4096, torch.bfloat16, 22))
    gv, gm = nm.pack(W, None, 2, 4)
    y1 = nm.spmv(gv, gm, x, 2, 4)
    y2 = nm.spmv(gv, gm, x, 2, 4)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_spmv_on_side_stream(nm):
    W = gpu(I.weight(256, 2048, torch.float16, 31))
    x = gpu(I.activation_normal(2, 2048, torch.float16, 32))
    gv, gm = nm.pack(W, None, 4, 8)
    ref = nm.spmv(gv, gm, x, 4, 8)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = nm.spmv(gv, gm, x, 4, 8)
    torch.cuda.current_stream().wait_stream(s)
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


# ---- dense baseline ------------------------------------------------------------

@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("R,K", [(1, 8), (45, 1000), (130, 4096), (16, 32768 + 512)])
@pytest.mark.parametrize("B", [1, 2, 8])
def test_gemv_dense(nm, dt, R, K, B):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("dW", R, K, dt))
    x = I.activation_normal(B, K, tdt, I.seed_of("dx", R, K, dt, B), outlier_frac=0.01)
    yref, A = oracle.gemv(bits(W), dt, bits(x))
    y = nm.gemv_dense(gpu(W), gpu(x))
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_gemv_dense_integer_exact(nm, dt):
    tdt = TD[dt]
    W = I.integer_valued(50, 3000 - 3000 % 8, tdt, 41, scale=1 / 16)
    x = I.integer_valued(3, W.shape[1], tdt, 42)
    yref, _ = oracle.gemv(bits(W), dt, bits(x))
    y = nm.gemv_dense(gpu(W), gpu(x))
    assert np.array_equal(bits(y), oracle.round_to(yref, dt))


# ---- several matrices sharing x in one launch -----------------------------------

@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
@pytest.mark.parametrize("Rs,K,B", [((96, 32, 32), 1024, 1), ((40, 0, 77, 13), 2048 + 16 * 3, 2),
                                     ((300, 300), 14336, 1), ((5,), 64, 8)])
def test_spmv_multi(nm, dt, n, m, Rs, K, B):
    tdt = TD[dt]
    x = I.activation_normal(B, K, tdt, I.seed_of("mx", K, B, dt), outlier_frac=0.01)
    parts, ref = [], []
    for i, R in enumerate(Rs):
        W = I.weight(R, K, tdt, I.seed_of("mW", i, R, K, dt, n, m))
        ov, om = oracle.pack(bits(W), None, n, m, dt)
        ref.append(oracle.spmv(ov, om, K, n, m, dt, bits(x)))
        parts.append(nm.pack(gpu(W), None, n, m))
    ys = nm.spmv_multi(parts, gpu(x), n, m)
    torch.cuda.synchronize()
    for i, (y, (yref, A)) in enumerate(zip(ys, ref)):
        assert y.shape == (B, Rs[i])
        ok, worst, idx = oracle.check(bits(y), yref, A, dt)
        assert ok, (i, worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_spmv_multi_integer_exact_matches_single(nm, dt):
    """Integer-valued inputs: every summation order is exact, so the fused
    launch must reproduce the single launches bit for bit."""
    tdt = TD[dt]
    K = 4096
    x = gpu(I.integer_valued(1, K, tdt, 51))
    parts = [nm.pack(gpu(I.integer_valued(R, K, tdt, 52 + R, scale=1 / 16)), None, 2, 4) for R in (256, 64, 64)]
    ys = nm.spmv_multi(parts, x, 2, 4)
    for (v, mk), y in zip(parts, ys):
        assert torch.equal(y.view(torch.int16), nm.spmv(v, mk, x, 2, 4).view(torch.int16))


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("Rs,K,B", [((64, 16, 16), 4096, 1), ((33, 70), 1000, 3)])
def test_gemv_dense_multi(nm, dt, Rs, K, B):
    tdt = TD[dt]
    x = I.activation_normal(B, K, tdt, I.seed_of("dmx", K, B, dt))
    Ws = [I.weight(R, K, tdt, I.seed_of("dmW", i, R, K, dt)) for i, R in enumerate(Rs)]
    ys = nm.gemv_dense_multi([gpu(W) for W in Ws], gpu(x))
    for W, y in zip(Ws, ys):
        yref, A = oracle.gemv(bits(W), dt, bits(x))
        ok, worst, idx = oracle.check(bits(y), yref, A, dt)
        assert ok, (worst, idx)


def test_spmv_very_long_rows(nm):
    """K = 2^20: x (2 MB) runs through the stream kernel in many K-tiles;
    the packed rows and every product against the oracle."""
    run_case(nm, 64, 1 << 20, 2, 4, "bf16", 1, seed=15)


@pytest.mark.parametrize("B", [2, 8])
def test_spmv_multi_tile_many_rows(nm, B):
    """Several x tiles with more rows than one pass of the grid's waves: the
    per-wave partial sums in LDS cover many rows."""
    run_case(nm, 5000, 25600, 2, 4, "bf16", B, seed=14)


@pytest.mark.parametrize("B", [3, 8])
def test_gemv_dense_multi_tile_many_rows(nm, B):
    tdt = torch.bfloat16
    R, K = 3000, 25600
    W = I.weight(R, K, tdt, I.seed_of("dmt", R, K, B))
    x = I.activation_normal(B, K, tdt, I.seed_of("dmtx", R, K, B))
    yref, A = oracle.gemv(bits(W), "bf16", bits(x))
    y = nm.gemv_dense(gpu(W), gpu(x))
    ok, worst, idx = oracle.check(bits(y), yref, A, "bf16")
    assert ok, (worst, idx)
