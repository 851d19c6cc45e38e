"""GPU parity of the K-split plan (nm_spmv_multi_ws, nm_gemv_dense_multi_ws):
batched products on few rows, where blocks of several 16-row tiles share one
staged x over one range of K and the last block of each tile group adds the
ranges' partial sums.  Every output element is checked against the oracle;
the workspace calls must also be deterministic, equal under graph replay,
and leave the workspace reusable for the next shape."""
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


@pytest.fixture(scope="module")
def ws(nm):
    return nm.workspace()


def bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def make(R, K, n, m, dt, B, seed):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("splitW", R, K, n, m, dt, seed))
    x = I.activation_normal(B, K, tdt, I.seed_of("splitx", R, K, dt, B, seed), outlier_frac=0.01)
    return W, x


def check_sparse(nm, ws, Ws, x, n, m, dt):
    """spmv_multi with the workspace over parts Ws against the oracle, element by element."""
    parts = [nm.pack(W.cuda(), None, n, m) for W in Ws]
    ys = nm.spmv_multi(parts, x.cuda(), n, m, ws=ws)
    torch.cuda.synchronize()
    worst = 0.0
    for W, y in zip(Ws, ys):
        ov, om = oracle.pack(bits(W), None, n, m, dt)
        yref, A = oracle.spmv(ov, om, W.shape[1], n, m, dt, bits(x))
        ok, w, idx = oracle.check(bits(y), yref, A, dt)
        assert ok, f"outside tolerance: worst ratio {w:.3f} at {idx}"
        worst = max(worst, w)
    return parts, ys, worst


# Few 16-row tiles and long rows (the shapes the K-split plan is for), ragged
# row counts and stage counts, one and two batch tiles, both formats.
@pytest.mark.parametrize("R,K,n,m,dt,B", [
    (320, 16384, 2, 4, "bf16", 8),
    (333, 16416, 2, 4, "fp16", 5),
    (300, 12288, 4, 8, "bf16", 16),
    (100, 25600, 2, 4, "bf16", 17),
    (250, 8192, 4, 8, "fp16", 32),
    (17, 32768, 2, 4, "fp16", 8),
    (5113, 4096, 2, 4, "bf16", 8),     # enough tiles for five units a block (one block a CU)
    (5113, 4096, 4, 8, "fp16", 16),
    (5113, 4096, 4, 8, "bf16", 32),
])
def test_splitk_sparse(nm, ws, R, K, n, m, dt, B):
    W, x = make(R, K, n, m, dt, B, 1)
    check_sparse(nm, ws, [W], x, n, m, dt)


def test_splitk_multi_parts(nm, ws):
    K, B = 14336, 8
    Ws = [make(R, K, 2, 4, "bf16", B, 10 + i)[0] for i, R in enumerate((130, 64, 97))]
    x = make(1, K, 2, 4, "bf16", B, 13)[1]
    check_sparse(nm, ws, Ws, x, 2, 4, "bf16")


@pytest.mark.parametrize("R,K,dt,B", [(320, 12800, "bf16", 8), (201, 8200, "fp16", 24)])
def test_splitk_dense(nm, ws, R, K, dt, B):
    W, x = make(R, K, 2, 4, dt, B, 2)
    y = nm.gemv_dense_multi([W.cuda()], x.cuda(), ws=ws)[0]
    torch.cuda.synchronize()
    yref, A = oracle.gemv(bits(W), dt, bits(x))
    ok, w, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (w, idx)


def test_splitk_deterministic_and_reusable(nm, ws):
    """The same call twice gives the same bits; a different shape in between
    (other tile groups, other split counts) leaves the workspace reusable."""
    W1, x1 = make(320, 16384, 2, 4, "bf16", 8, 3)
    W2, x2 = make(96, 25600, 2, 4, "bf16", 16, 4)
    p1 = [nm.pack(W1.cuda(), None, 2, 4)]
    p2 = [nm.pack(W2.cuda(), None, 2, 4)]
    a = nm.spmv_multi(p1, x1.cuda(), 2, 4, ws=ws)[0].clone()
    nm.spmv_multi(p2, x2.cuda(), 2, 4, ws=ws)
    b = nm.spmv_multi(p1, x1.cuda(), 2, 4, ws=ws)[0].clone()
    fresh = nm.workspace()
    c = nm.spmv_multi(p1, x1.cuda(), 2, 4, ws=fresh)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_splitk_graph_replay(nm, ws):
    """Captured into a HIP graph, every replay (with eager calls on the same
    workspace between them) equals the eager result bit for bit."""
    W, x = make(320, 16384, 2, 4, "fp16", 8, 5)
    parts = [nm.pack(W.cuda(), None, 2, 4)]
    xc = x.cuda()
    eager = nm.spmv_multi(parts, xc, 2, 4, ws=ws)[0].clone()
    Wo, xo = make(160, 25600, 2, 4, "fp16", 16, 6)
    other = [nm.pack(Wo.cuda(), None, 2, 4)]
    xoc = xo.cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        out = nm.spmv_multi(parts, xc, 2, 4, stream=s, ws=ws)[0]
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            out = nm.spmv_multi(parts, xc, 2, 4, stream=s, ws=ws)[0]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        nm.spmv_multi(other, xoc, 2, 4, ws=ws)           # other work on the same workspace between replays
        torch.cuda.synchronize()


def test_workspace_argument_checks(nm, ws):
    W, x = make(64, 4096, 2, 4, "fp16", 8, 7)
    parts = [nm.pack(W.cuda(), None, 2, 4)]
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        nm.spmv_multi(parts, x.cuda(), 2, 4, ws=ws[:-1])             # one byte short
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        nm.spmv_multi(parts, x.cuda(), 2, 4, ws=ws[16:])             # not 256-byte aligned
