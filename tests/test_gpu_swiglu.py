"""GPU parity of the gated-MLP launch: h = SiLU(W_gate x) * (W_up x) from
``nm_spmv_swiglu`` (packed N:M gate and up) and ``nm_gemv_dense_swiglu`` (dense),
through the C ABI, against the oracle's exact sums and its SiLU.  The bound
(oracle.swiglu_tolerance) propagates the product rule's error of each sum
through SiLU (Lipschitz 1.1) and the multiply, plus the fp32 evaluation and
one ulp of the output format; with integer-valued operands the sums are exact
and only the evaluation and rounding remain."""
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
    rows = {0, R // 2, R - 1} | set(g.choice(R, size=min(k, R), replace=False).tolist())
    return sorted(rows)


def run_sparse(nm, R, K, n, m, dt, B, seed, rows=None, integer=False, device_inputs=False):
    tdt = TD[dt]
    dev = "cuda" if device_inputs else "cpu"
    if integer:
        Wg = I.integer_valued(R, K, tdt, I.seed_of("glu_g", R, K, n, m, dt, seed), scale=1 / 16, device=dev)
        Wu = I.integer_valued(R, K, tdt, I.seed_of("glu_u", R, K, n, m, dt, seed), scale=1 / 16, device=dev)
        x = I.integer_valued(B, K, tdt, I.seed_of("glu_x", R, K, dt, B, seed), lo=-3, hi=3, device=dev)
    else:
        Wg = I.weight(R, K, tdt, I.seed_of("glu_g", R, K, n, m, dt, seed), device=dev)
        Wu = I.weight(R, K, tdt, I.seed_of("glu_u", R, K, n, m, dt, seed), device=dev)
        x = I.activation_normal(B, K, tdt, I.seed_of("glu_x", R, K, dt, B, seed), device=dev, outlier_frac=0.01)
    g = nm.pack(Wg.cuda(), None, n, m)
    u = nm.pack(Wu.cuda(), None, n, m)
    h = nm.spmv_swiglu(g, u, x.cuda(), n, m)
    torch.cuda.synchronize()
    assert h.shape == (B, R)
    rows = list(range(R)) if rows is None else rows
    xb = bits(x)
    gv, gm = oracle.pack(bits(Wg[rows]), None, n, m, dt)
    uv, um = oracle.pack(bits(Wu[rows]), None, n, m, dt)
    assert np.array_equal(bits(g[0][rows]), gv) and np.array_equal(g[1][rows].cpu().numpy(), gm)
    gref, Ag = oracle.spmv(gv, gm, K, n, m, dt, xb)
    uref, Au = oracle.spmv(uv, um, K, n, m, dt, xb)
    ok, worst, idx = oracle.check_swiglu(bits(h[:, rows]), gref, uref, Ag, Au, dt, exact_sums=integer)
    assert ok, f"swiglu outside tolerance: worst ratio {worst:.3f} at {idx}"
    return worst


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
@pytest.mark.parametrize("R,K", [(1, 16), (7, 80), (130, 1040), (515, 4096)])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_swiglu_sparse(nm, dt, n, m, R, K, B):
    run_sparse(nm, R, K, n, m, dt, B, seed=1)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
@pytest.mark.parametrize("B", [1, 8])
def test_swiglu_integer_exact_sums(nm, dt, n, m, B):
    """Integer-valued operands: g and u are exact in fp32 whatever the order,
    so h may differ from the oracle's only by the fp32 SiLU/multiply and the
    final rounding."""
    run_sparse(nm, 77, 2048 + 64, n, m, dt, B, seed=2, integer=True)


@pytest.mark.parametrize("n,m,K", [(1, 4, 24), (3, 4, 72), (1, 8, 40), (5, 8, 1000), (2, 4, 24), (4, 8, 1032)])
@pytest.mark.parametrize("B", [1, 5])
def test_swiglu_any_nm(nm, n, m, K, B):
    """Patterns and widths outside the fast 2:4 / 4:8, K % 16 == 0 path (one
    wave per output row reduces both matrices)."""
    run_sparse(nm, 45, K, n, m, "bf16", B, seed=3)


@pytest.mark.parametrize("R,K,B", [(600, 28672, 1), (700, 8192, 8), (3000, 25600, 4)])
def test_swiglu_stream_kernel(nm, R, K, B):
    """x beyond the row-slice LDS budget: the stream kernel takes the row
    pairs, with one x tile (K = 28672, B = 1) or several (the others)."""
    run_sparse(nm, R, K, 2, 4, "bf16", B, seed=4, rows=sample_rows(R, 5))


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("R,K,B", [(9, 64, 1), (300, 4096, 2), (64, 14336, 8)])
def test_swiglu_dense(nm, dt, R, K, B):
    tdt = TD[dt]
    Wg = I.weight(R, K, tdt, I.seed_of("dglu_g", R, K, dt))
    Wu = I.weight(R, K, tdt, I.seed_of("dglu_u", R, K, dt))
    x = I.activation_normal(B, K, tdt, I.seed_of("dglu_x", R, K, dt, B))
    h = nm.gemv_dense_swiglu(Wg.cuda(), Wu.cuda(), x.cuda())
    gref, Ag = oracle.gemv(bits(Wg), dt, bits(x))
    uref, Au = oracle.gemv(bits(Wu), dt, bits(x))
    ok, worst, idx = oracle.check_swiglu(bits(h), gref, uref, Ag, Au, dt)
    assert ok, (worst, idx)


def test_swiglu_empty_and_degenerate(nm):
    tdt = torch.float16
    # K == 0: SiLU(0) * 0 = 0
    e = torch.empty((5, 0), dtype=tdt, device="cuda")
    em = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    h = torch.full((2, 5), 7, dtype=tdt, device="cuda")
    nm.spmv_swiglu((e, em), (e, em), torch.empty((2, 0), dtype=tdt, device="cuda"), 2, 4, out=h)
    assert torch.all(h == 0)
    # R == 0
    v = torch.empty((0, 32), dtype=tdt, device="cuda")
    mk = torch.empty((0, 8), dtype=torch.uint8, device="cuda")
    assert nm.spmv_swiglu((v, mk), (v, mk), torch.ones((3, 64), dtype=tdt, device="cuda"), 2, 4).shape == (3, 0)
    # a zero gate gives h = 0 whatever the up product is
    Wg = torch.zeros((70, 64), dtype=tdt, device="cuda")
    Wu = torch.ones((70, 64), dtype=tdt, device="cuda")
    h = nm.spmv_swiglu(nm.pack(Wg, None, 2, 4), nm.pack(Wu, None, 2, 4), torch.ones((1, 64), dtype=tdt, device="cuda"))
    assert torch.all(h == 0)


@pytest.mark.parametrize("shape", ["llama31_8b", "qwen3_32b_b8"])
def test_swiglu_full_size(nm, shape):
    """Full MLP input shapes in the launch configuration the benchmark uses:
    Llama-3.1-8B gate/up 14336 x 4096 (2:4 fp16, B = 1) and Qwen3-32B 25600 x
    5120 (2:4 bf16, B = 8, x in several tiles); sampled rows."""
    if shape == "llama31_8b":
        R, K, dt, B = 14336, 4096, "fp16", 1
    else:
        R, K, dt, B = 25600, 5120, "bf16", 8
    run_sparse(nm, R, K, 2, 4, dt, B, seed=6, rows=sample_rows(R, 7, k=20), device_inputs=True)
