"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark uses.  Weights and activations are drawn on the GPU (seeded); the
oracle checks every row: packed bytes identical, products within the
acceptance bound, the rows split over the host's threads (the C oracle runs
outside Python's lock).

Workloads: Llama-3.1-8B projections (2:4 fp16, x with 1% outlier channels,
single and fused q+k+v / gate+up launches), Qwen3-14B/32B MLP (4:8 and 2:4
bf16, Laplace x), one Llama-3.3-70B layer (2:4 bf16), Qwen3-32B MLP at batch
1/2/4/8/16/32 (2:4 bf16), and the dense baseline on the same rows."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from sparse_matrix_vector_amd import inputs as I

pytestmark = pytest.mark.gpu

TD = {"fp16": torch.float16, "bf16": torch.bfloat16}
NTHREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def nm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_matrix_vector_amd as nm
    nm.lib()
    return nm


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def check_all_rows(W, values, masks, x, y, n, m, dt, yd=None, y_more=(), yd_more=()):
    """Every row of the packed matrix, the sparse product and (given yd) the
    dense product against the oracle, in row ranges over NTHREADS threads;
    y_more / yd_more: further sparse / dense products of the same inputs
    (other calls), checked against the same oracle results."""
    Wb, vb, mb, xb, yb = bits(W), bits(values), masks.cpu().numpy(), bits(x), bits(y)
    ydb = None if yd is None else bits(yd)
    ymb = [bits(t) for t in y_more]
    ydmb = [bits(t) for t in yd_more]
    R, K = Wb.shape
    step = max(1, -(-R // (4 * NTHREADS)))

    def job(r0):
        r1 = min(R, r0 + step)
        ov, om = oracle.pack(Wb[r0:r1], None, n, m, dt)
        if not np.array_equal(vb[r0:r1], ov):
            return f"packed values differ in rows {r0}..{r1 - 1}"
        if not np.array_equal(mb[r0:r1], om):
            return f"masks differ in rows {r0}..{r1 - 1}"
        yref, A = oracle.spmv(ov, om, K, n, m, dt, xb)
        for j, yy in enumerate([yb] + ymb):
            ok, worst, idx = oracle.check(yy[:, r0:r1], yref, A, dt)
            if not ok:
                return f"spmv (output {j}) outside tolerance in rows {r0}..{r1 - 1}: worst {worst:.3f} at {idx}"
        if ydb is not None or ydmb:
            ydref, Ad = oracle.gemv(Wb[r0:r1], dt, xb)
            for j, yy in enumerate(([ydb] if ydb is not None else []) + ydmb):
                ok, worst, idx = oracle.check(yy[:, r0:r1], ydref, Ad, dt)
                if not ok:
                    return f"dense gemv (output {j}) outside tolerance in rows {r0}..{r1 - 1}: worst {worst:.3f} at {idx}"
        return None

    with ThreadPoolExecutor(NTHREADS) as ex:
        for err in ex.map(job, range(0, R, step)):
            assert err is None, err


def make(R, K, dt, tag, B=1, xkind="normal"):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of(tag, "W"), device="cuda")
    if xkind == "laplace":
        x = I.activation_laplace(B, K, tdt, I.seed_of(tag, "x"), device="cuda")
    else:
        x = I.activation_normal(B, K, tdt, I.seed_of(tag, "x"), device="cuda",
                                outlier_frac=0.01 if xkind == "outliers" else 0.0)
    return W, x


@pytest.fixture(scope="module")
def ws(nm):
    return nm.workspace()


def ws_products(nm, ws, W, v, mk, x, n, m, dense=True):
    """The same products through the workspace calls (the benchmark's steps
    use them; long rows there take the K-split plans)."""
    yw = nm.spmv_multi([(v, mk)], x, n, m, ws=ws)[0]
    ydw = nm.gemv_dense_multi([W], x, ws=ws)[0] if dense else None
    return (yw,), ((ydw,) if dense else ())


@pytest.mark.parametrize("name", list(I.LLAMA31_8B))
def test_llama31_8b_single(nm, ws, name):
    R, K = I.LLAMA31_8B[name]
    W, x = make(R, K, "fp16", ("llama31_8b", name), xkind="outliers")
    v, mk = nm.pack(W, None, 2, 4)
    y = nm.spmv(v, mk, x, 2, 4)
    yd = nm.gemv_dense(W, x)
    ym, ydm = ws_products(nm, ws, W, v, mk, x, 2, 4)
    torch.cuda.synchronize()
    check_all_rows(W, v, mk, x, y, 2, 4, "fp16", yd, y_more=ym, yd_more=ydm)


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
        check_all_rows(W, v, mk, x, y, 2, 4, "fp16", yd)


@pytest.mark.parametrize("model,shapes", [("qwen3_14b", I.QWEN3_14B_MLP), ("qwen3_32b", I.QWEN3_32B_MLP)])
@pytest.mark.parametrize("n,m", [(4, 8), (2, 4)])
def test_qwen3_mlp(nm, ws, model, shapes, n, m):
    for name, (R, K) in shapes.items():
        W, x = make(R, K, "bf16", (model, name, n, m), xkind="laplace")
        v, mk = nm.pack(W, None, n, m)
        y = nm.spmv(v, mk, x, n, m)
        yd = nm.gemv_dense(W, x) if name != "up" else None
        ym, ydm = ws_products(nm, ws, W, v, mk, x, n, m, dense=name != "up")
        torch.cuda.synchronize()
        check_all_rows(W, v, mk, x, y, n, m, "bf16", yd, y_more=ym, yd_more=ydm)
        del W, v, mk


@pytest.mark.parametrize("name", list(I.LLAMA33_70B))
def test_llama33_70b_layer(nm, ws, name):
    R, K = I.LLAMA33_70B[name]
    W, x = make(R, K, "bf16", ("llama33_70b", 0, name))
    v, mk = nm.pack(W, None, 2, 4)
    y = nm.spmv(v, mk, x, 2, 4)
    yd = nm.gemv_dense(W, x) if name in ("q", "down") else None
    ym, ydm = ws_products(nm, ws, W, v, mk, x, 2, 4, dense=name in ("q", "down"))
    torch.cuda.synchronize()
    check_all_rows(W, v, mk, x, y, 2, 4, "bf16", yd, y_more=ym, yd_more=ydm)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_qwen3_32b_small_batch(nm, B):
    """Each batch size bench.py times at the Qwen3-32B MLP shapes, through the
    plain calls and through the workspace calls the benchmark's steps use
    (down from 4 vectors: the K-split plan, five tile units a block; 16 and
    32 two tiles a wave, 32 two batch tiles; plain down above 16: the staged
    kernel)."""
    ws = nm.workspace()
    for name, (R, K) in I.QWEN3_32B_MLP.items():
        W, x = make(R, K, "bf16", ("qwen3_32b_batch", name, B), B=B)
        v, mk = nm.pack(W, None, 2, 4)
        y = nm.spmv(v, mk, x, 2, 4)
        yd = nm.gemv_dense(W, x)
        yw = nm.spmv_multi([(v, mk)], x, 2, 4, ws=ws)[0]
        ydw = nm.gemv_dense_multi([W], x, ws=ws)[0]
        torch.cuda.synchronize()
        assert y.shape == (B, R) and yw.shape == (B, R)
        check_all_rows(W, v, mk, x, y, 2, 4, "bf16", yd, y_more=(yw,), yd_more=(ydw,))
        del W, v, mk


def test_tiny_1024_seed0_full(nm):
    """The 1024 x 1024 case checked in full (every row), W from seed 0 on the CPU."""
    W = I.weight(1024, 1024, torch.float16, 0)
    x = I.activation_normal(1, 1024, torch.float16, I.seed_of("x", 0))
    v, mk = nm.pack(W.cuda(), None, 2, 4)
    y = nm.spmv(v, mk, x.cuda(), 2, 4)
    check_all_rows(W, v, mk, x, y, 2, 4, "fp16")


def test_spmv_x_past_2g_units(nm):
    """32 vectors of K = 671088640 (x is 43 GB; the last row starts
    31 K / 8 > 2^31 16-byte units in) over 16 rows, which the staged
    matrix-core kernel takes.  The packed operands are built on the GPU
    (columns 0 and 1 of every group kept, seeded values) and every x row is
    the same seeded row: all 32 outputs of a row bit-identical, finite and
    not all zero, a second call bit-identical to the first, and the first and
    last rows within the acceptance bound of the oracle's."""
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
    # rows 0 and 15 against the oracle (one row of values is 671 MB, x is one 1.3 GB row)
    xb = bits(x[:1])
    for r in (0, R - 1):
        yref, A = oracle.spmv(bits(values[r:r + 1]), masks[r:r + 1].cpu().numpy(), K, 2, 4, "bf16", xb)
        ok, worst, idx = oracle.check(bits(y[:, r:r + 1]), np.repeat(yref, B, axis=0), np.repeat(A, B, axis=0), "bf16")
        assert ok, f"row {r}: worst {worst:.3f} at {idx}"
    del values, masks, x, y, y2
    torch.cuda.empty_cache()
