"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark uses.  Weights and activations are drawn on the GPU (seeded); the
oracle checks sampled rows one by one: their packed bytes must be identical
and their products within the acceptance bound.

Workloads: Llama-3.1-8B projections (2:4 fp16, x with 1% outlier channels,
single and fused q+k+v / gate+up launches), Qwen3-14B/32B MLP (4:8 and 2:4
bf16, Laplace x), one Llama-3.3-70B layer (2:4 bf16), Qwen3-32B MLP at batch
1/2/4/8 (2:4 bf16), and the dense baseline on the same rows."""
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


def sample_rows(R, seed, k=24):
    g = np.random.default_rng(seed)
    rows = set([0, 1, R // 2, R - 2, R - 1]) | set(g.choice(R, size=min(k, R), replace=False).tolist())
    return sorted(r for r in rows if 0 <= r < R)


def check_rows(W, values, masks, x, y, n, m, dt, rows, yd=None):
    xb = bits(x)
    Wb = bits(W[rows])
    ov, om = oracle.pack(Wb, None, n, m, dt)
    assert np.array_equal(bits(values[rows]), ov), "packed values differ on sampled rows"
    assert np.array_equal(masks[rows].cpu().numpy(), om), "masks differ on sampled rows"
    yref, A = oracle.spmv(ov, om, W.shape[1], n, m, dt, xb)
    ok, worst, idx = oracle.check(bits(y[:, rows]), yref, A, dt)
    assert ok, f"spmv outside tolerance: worst {worst:.3f} at {idx}"
    if yd is not None:
        ydref, Ad = oracle.gemv(Wb, dt, xb)
        ok, worst, idx = oracle.check(bits(yd[:, rows]), ydref, Ad, dt)
        assert ok, f"dense gemv outside tolerance: worst {worst:.3f} at {idx}"


def make(R, K, dt, tag, B=1, xkind="normal"):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of(tag, "W"), device="cuda")
    if xkind == "laplace":
        x = I.activation_laplace(B, K, tdt, I.seed_of(tag, "x"), device="cuda")
    else:
        x = I.activation_normal(B, K, tdt, I.seed_of(tag, "x"), device="cuda",
                                outlier_frac=0.01 if xkind == "outliers" else 0.0)
    return W, x


@pytest.mark.parametrize("name", list(I.LLAMA31_8B))
def test_llama31_8b_single(nm, name):
    R, K = I.LLAMA31_8B[name]
    W, x = make(R, K, "fp16", ("llama31_8b", name), xkind="outliers")
    v, mk = nm.pack(W, None, 2, 4)
    y = nm.spmv(v, mk, x, 2, 4)
    yd = nm.gemv_dense(W, x)
    torch.cuda.synchronize()
    check_rows(W, v, mk, x, y, 2, 4, "fp16", sample_rows(R, 1), yd)


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_llama31_8b_fused(nm, group):
    K = I.LLAMA31_8B[group[0]][1]
    x = I.activation_normal(1, K, torch.float16, I.seed_of("fused", group), device="cuda", outlier_frac=0.01)
    Ws = [I.weight(*I.LLAMA31_8B[g], torch.float16, I.seed_of("fused", g), device="cuda") for g in group]
    parts = [nm.pack(W, None, 2, 4) for W in Ws]
    ys = nm.spmv_multi(parts, x, 2, 4)
    yds = nm.gemv_dense_multi(Ws, x)
    torch.cuda.synchronize()
    for W, (v, mk), y, yd in zip(Ws, parts, ys, yds):
        check_rows(W, v, mk, x, y, 2, 4, "fp16", sample_rows(W.shape[0], 2), yd)


@pytest.mark.parametrize("model,shapes", [("qwen3_14b", I.QWEN3_14B_MLP), ("qwen3_32b", I.QWEN3_32B_MLP)])
@pytest.mark.parametrize("n,m", [(4, 8), (2, 4)])
def test_qwen3_mlp(nm, model, shapes, n, m):
    for name, (R, K) in shapes.items():
        W, x = make(R, K, "bf16", (model, name, n, m), xkind="laplace")
        v, mk = nm.pack(W, None, n, m)
        y = nm.spmv(v, mk, x, n, m)
        yd = nm.gemv_dense(W, x) if name != "up" else None
        torch.cuda.synchronize()
        check_rows(W, v, mk, x, y, n, m, "bf16", sample_rows(R, 3, k=12), yd)
        del W, v, mk


@pytest.mark.parametrize("name", list(I.LLAMA33_70B))
def test_llama33_70b_layer(nm, name):
    R, K = I.LLAMA33_70B[name]
    W, x = make(R, K, "bf16", ("llama33_70b", 0, name))
    v, mk = nm.pack(W, None, 2, 4)
    y = nm.spmv(v, mk, x, 2, 4)
    yd = nm.gemv_dense(W, x) if name in ("q", "down") else None
    torch.cuda.synchronize()
    check_rows(W, v, mk, x, y, 2, 4, "bf16", sample_rows(R, 4, k=12), yd)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_qwen3_32b_small_batch(nm, B):
    """Each batch size bench.py times at the Qwen3-32B MLP shapes; 16 and 32
    run the matrix-core kernels in their large-batch shapes (gate/up: two
    waves of two tiles sharing x, two batch tiles; down: the staged kernel
    above 16)."""
    for name, (R, K) in I.QWEN3_32B_MLP.items():
        W, x = make(R, K, "bf16", ("qwen3_32b_batch", name, B), B=B)
        v, mk = nm.pack(W, None, 2, 4)
        y = nm.spmv(v, mk, x, 2, 4)
        yd = nm.gemv_dense(W, x)
        torch.cuda.synchronize()
        assert y.shape == (B, R)
        check_rows(W, v, mk, x, y, 2, 4, "bf16", sample_rows(R, 5, k=10), yd)
        del W, v, mk


def test_tiny_1024_seed0_full(nm):
    """The 1024 x 1024 case checked in full (every row), W from seed 0 on the CPU."""
    W = I.weight(1024, 1024, torch.float16, 0)
    x = I.activation_normal(1, 1024, torch.float16, I.seed_of("x", 0))
    v, mk = nm.pack(W.cuda(), None, 2, 4)
    y = nm.spmv(v, mk, x.cuda(), 2, 4)
    check_rows(W, v.cpu(), mk.cpu(), x, y.cpu(), 2, 4, "fp16", list(range(1024)))


def test_spmv_x_past_2g_units(nm):
    """32 vectors of K = 671088640 (x is 43 GB; the last row starts
    31 K / 8 > 2^31 16-byte units in) over 16 rows, which the staged
    matrix-core kernel takes.  Too large for the oracle, so the packed
    operands are built on the GPU (columns 0 and 1 of every group kept,
    seeded values) and every x row is the same seeded row; properties that
    hold at any size: all 32 outputs of a row bit-identical, finite and not
    all zero, and a second call bit-identical to the first."""
    R, K, B = 16, 671088640, 32
    need = B * K * 2 + R * (K // 2) * 6 + R * (K // 8) + (2 << 30)
    if torch.cuda.mem_get_info()[0] < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory")
    g = torch.Generator(device="cuda")
    g.manual_seed(I.seed_of("xbig", R, K, B))
    values = torch.empty((R, K // 2), dtype=torch.bfloat16, device="cuda")
    for r in range(R):                        # one row at a time keeps the fp32 draw small
        values[r] = (torch.randn(K // 2, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    masks = torch.full((R, K // 8), 0x33, dtype=torch.uint8, device="cuda")
    x0 = torch.randn(K, device="cuda", generator=g).to(torch.bfloat16)
    x = x0.expand(B, K).contiguous()
    del x0
    y = nm.spmv(values, masks, x, 2, 4)
    y2 = nm.spmv(values, masks, x, 2, 4)
    torch.cuda.synchronize()
    assert y.shape == (B, R)
    yb = y.view(torch.int16)
    assert torch.equal(yb, yb[:1].expand(B, R)), "batch columns differ"
    assert torch.isfinite(y.float()).all() and (y[0] != 0).any()
    assert torch.equal(yb, y2.view(torch.int16))
    del values, masks, x, y, y2
    torch.cuda.empty_cache()
