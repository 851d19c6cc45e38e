"""GPU parity of the hybrid sparse + dense row format through the C ABI:
the per-row pruning loss and the dense-row choice bit for bit against the
oracle (both sum in double in the same order), the packed parts and row lists
byte for byte, and the hybrid product within the product rule's bound against
the oracle's sparse rows plus dense rows."""
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


def random_keep(R, K, n, m, seed):
    return I.keep_mask(R, K, n, m, seed)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4)])
@pytest.mark.parametrize("mode", ["magnitude", "keep", "calibrated"])
def test_row_loss_and_choice_bitexact(nm, dt, n, m, mode):
    R, K = 300, 1040
    W = I.weight(R, K, TD[dt], I.seed_of("hyW", dt, n, m))
    W = (torch.round(W.float() / 0.004) * 0.004).to(TD[dt])        # equal magnitudes: ties in the keep rule
    keep = random_keep(R, K, n, m, I.seed_of("hyK", n, m)) if mode == "keep" else None
    h = None
    if mode == "calibrated":
        h = (np.random.default_rng(I.seed_of("hyh", dt)).random(K) * 3).astype(np.float32)
        h[:5] = [0.0, 1e-40, 2.5e38, 1.0, 1.0]
    loss = nm.hybrid_row_loss(W.cuda(), n, m, keep=None if keep is None else keep.cuda(),
                              H=None if h is None else torch.from_numpy(h).cuda())
    want = oracle.hybrid_row_loss(bits(W), n, m, dt, keep=None if keep is None else keep.numpy(), h=h)
    assert np.array_equal(loss.cpu().numpy(), want)
    for nd in (0, 1, 37, R):
        flags = nm.hybrid_select_rows(loss, nd)
        assert np.array_equal(flags.cpu().numpy(), oracle.hybrid_select(want, nd))


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("with_keep", [False, True])
def test_row_loss_unaligned_inputs(nm, dt, with_keep):
    """W 2 bytes and keep 1 byte past an aligned address (the call accepts
    both): rows are then staged element by element, with the same sums."""
    R, K, n, m = 300, 1040, 2, 4
    W = I.weight(R, K, TD[dt], I.seed_of("hyU", dt))
    buf = torch.empty(R * K + 8, dtype=TD[dt], device="cuda")
    Wu = buf[1:1 + R * K].view(R, K)
    Wu.copy_(W.cuda())
    keep = kp = None
    if with_keep:
        keep = random_keep(R, K, n, m, I.seed_of("hyUk"))
        kbuf = torch.empty(R * K + 16, dtype=torch.uint8, device="cuda")
        kp = kbuf[1:1 + R * K].view(R, K)
        kp.copy_(keep.cuda())
    assert Wu.data_ptr() % 16 != 0 and (kp is None or kp.data_ptr() % 8 != 0)
    loss = nm.hybrid_row_loss(Wu, n, m, keep=kp)
    want = oracle.hybrid_row_loss(bits(W), n, m, dt, keep=None if keep is None else keep.numpy())
    assert np.array_equal(loss.cpu().numpy(), want)


@pytest.mark.parametrize("values", [
    [3.0, 1.0, 3.0, float("nan"), 0.0, 7.0, 1.0, 3.0],
    [-5.0, float("nan"), -0.5, 2.0, -float("inf"), -5.0, float("nan"), -1.0],   # NaN below negatives and -inf
    [float("nan"), -float("inf")],                                                 # -inf chosen before NaN ...
    [-float("inf"), float("nan")],                                                 # ... in either order
    [float("nan"), -float("inf"), float("nan"), -float("inf"), float("inf"), -0.0, 0.0, float("nan")],
])
def test_row_choice_ties_and_nan(nm, values):
    loss = torch.tensor(values, dtype=torch.float64)
    for nd in range(loss.numel() + 1):
        got = nm.hybrid_select_rows(loss.cuda(), nd).cpu().numpy()
        assert np.array_equal(got, oracle.hybrid_select(loss.numpy(), nd)), nd


def test_row_choice_many_rows_all_partitions(nm):
    """1000 rows (16 blocks, the last partial), many equal losses, NaNs and
    negatives: every count of dense rows matches the oracle."""
    g = np.random.default_rng(21)
    loss = np.round(g.normal(0, 2, 1000), 1)
    loss[g.random(1000) < 0.05] = np.nan
    lt = torch.from_numpy(loss).cuda()
    for nd in (0, 1, 63, 64, 65, 500, 999, 1000):
        got = nm.hybrid_select_rows(lt, nd).cpu().numpy()
        assert np.array_equal(got, oracle.hybrid_select(loss, nd)), nd


def test_row_loss_errors(nm):
    W = I.weight(8, 64, torch.float16, 3).cuda()
    W[2, 5] = float("nan")
    with pytest.raises(nm.NmError) as e:
        nm.hybrid_row_loss(W, 2, 4)
    assert e.value.status == nm.NM_ERR_NONFINITE
    bad = torch.ones((8, 64), dtype=torch.uint8, device="cuda")      # 4 kept per group, not 2
    with pytest.raises(nm.NmError) as e:
        nm.hybrid_row_loss(W, 2, 4, keep=bad)
    assert e.value.status == nm.NM_ERR_BAD_MASK


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m,K", [(2, 4, 1040), (4, 8, 4096), (1, 4, 72)])
@pytest.mark.parametrize("B", [1, 3, 8, 20])
@pytest.mark.parametrize("frac", [0.0, 0.1, 1.0])
def test_hybrid_pack_and_spmv(nm, dt, n, m, K, B, frac):
    R = 130
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("hpW", dt, n, m, K))
    x = I.activation_normal(B, K, tdt, I.seed_of("hpx", dt, K, B), outlier_frac=0.01)
    nd = int(round(frac * R))
    loss = nm.hybrid_row_loss(W.cuda(), n, m)
    flags = nm.hybrid_select_rows(loss, nd)
    hyb = nm.hybrid_pack(W.cuda(), flags, nd, n, m)
    f = flags.cpu().numpy().astype(bool)
    assert np.array_equal(hyb.rows_dense.cpu().numpy(), np.nonzero(f)[0])
    assert np.array_equal(hyb.rows_sparse.cpu().numpy(), np.nonzero(~f)[0])
    assert np.array_equal(bits(hyb.W_dense), bits(W)[f])
    if (~f).any():
        ov, om = oracle.pack(bits(W)[~f], None, n, m, dt)
        assert np.array_equal(bits(hyb.values), ov) and np.array_equal(hyb.masks.cpu().numpy(), om)
    y = nm.spmv_hybrid(hyb, x.cuda())
    yref, A = oracle.hybrid_spmv(bits(W), f, n, m, dt, bits(x))
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)


# Shapes (at one to three vectors) whose sparse and dense rows run in one launch: one
# slice (K = 1040, 4096), two (K = 8192; dense rows at four), four (K = 18432,
# or few rows; dense rows at eight, one per block); few sparse rows (taken two
# per block); ragged row counts on both sides.
@pytest.mark.parametrize("dt,n,m,K,R,frac", [
    ("fp16", 2, 4, 1040, 4097, 0.1),
    ("bf16", 4, 8, 4096, 4096, 0.05),
    ("bf16", 2, 4, 8192, 4100, 0.5),
    ("fp16", 4, 8, 8192, 3001, 0.3),
    ("fp16", 2, 4, 18432, 2100, 0.25),
    ("fp16", 2, 4, 4096, 1024, 0.05),           # few sparse rows: two per block in the one launch
    ("bf16", 4, 8, 1040, 600, 0.2),
    ("bf16", 2, 4, 25600, 700, 0.1),            # the longest rows on the row-slice kernel: 4 slices, 8 for dense
])
@pytest.mark.parametrize("B", [1, 2, 3])
def test_hybrid_one_launch_shapes(nm, dt, n, m, K, R, frac, B):
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("h1W", dt, n, m, K, R), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("h1x", dt, K, B), device="cuda", outlier_frac=0.01)
    nd = int(round(frac * R))
    flags = nm.hybrid_select_rows(nm.hybrid_row_loss(W, n, m), nd)
    hyb = nm.hybrid_pack(W, flags, nd, n, m)
    y = nm.spmv_hybrid(hyb, x)
    f = flags.cpu().numpy().astype(bool)
    yref, A = oracle.hybrid_spmv(bits(W), f, n, m, dt, bits(x))
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)


@pytest.mark.parametrize("R,K,B", [(4097, 1040, 1), (130, 1040, 2)])   # one launch; two launches
def test_hybrid_bad_row_lists_stay_inside_y(nm, R, K, B):
    """Row lists that do not partition 0..R-1 leave y unspecified, but every
    entry is clamped into 0..R-1: rows out of range on both lists (past R,
    negative) write inside y, never past it.  y is the front of a larger
    buffer whose tail must keep its sentinel; rows the lists still map
    correctly, and that no clamped entry lands on, hold their products."""
    dt, tdt, n, m = "fp16", torch.float16, 2, 4
    W = I.weight(R, K, tdt, I.seed_of("hbW", R), device="cuda")
    x = I.activation_normal(B, K, tdt, I.seed_of("hbx", R, B), device="cuda")
    nd = R // 10
    flags = nm.hybrid_select_rows(nm.hybrid_row_loss(W, n, m), nd)
    hyb = nm.hybrid_pack(W, flags, nd, n, m)
    rs, rd = hyb.rows_sparse.cpu().numpy().copy(), hyb.rows_dense.cpu().numpy().copy()
    hyb.rows_sparse[1] = R + 100                   # clamps to R - 1
    hyb.rows_sparse[2] = -7                        # clamps to 0
    hyb.rows_dense[0] = 1 << 30                    # clamps to R - 1
    big = torch.full((B * R + 256,), 12345.0, dtype=tdt, device="cuda")
    nm.spmv_hybrid(hyb, x, out=big[:B * R].view(B, R))
    assert torch.all(big[B * R:].cpu() == 12345.0)
    f = flags.cpu().numpy().astype(bool)
    yref, A = oracle.hybrid_spmv(bits(W), f, n, m, dt, bits(x))
    touched = {0, R - 1, int(rs[1]), int(rs[2]), int(rd[0])}
    keep = np.array([r for r in range(R) if r not in touched])
    y = bits(big[:B * R].view(B, R))
    ok, worst, idx = oracle.check(y[:, keep], yref[:, keep], A[:, keep], dt)
    assert ok, (worst, idx)


def test_hybrid_with_calibrated_keep(nm):
    """The two offline pieces together: a calibration keep-mask drives both
    the sparse rows' pattern and the loss that picks the dense rows."""
    R, K, T, dt = 256, 2048, 64, "bf16"
    W = I.weight(R, K, torch.bfloat16, I.seed_of("hcW")).cuda()
    X = I.activation_normal(T, K, torch.bfloat16, I.seed_of("hcX"), device="cuda", outlier_frac=0.01)
    H = nm.calib_accumulate(X)
    keep = nm.calib_keep_mask(W, H, 2, 4)
    loss = nm.hybrid_row_loss(W, 2, 4, keep=keep, H=H)
    hdiag = torch.diagonal(H).contiguous().cpu().numpy()
    want = oracle.hybrid_row_loss(bits(W), 2, 4, dt, keep=keep.cpu().numpy(), h=hdiag)
    assert np.array_equal(loss.cpu().numpy(), want)
    flags = nm.hybrid_select_rows(loss, 32)
    hyb = nm.hybrid_pack(W, flags, 32, 2, 4, keep=keep)
    x = I.activation_normal(2, K, torch.bfloat16, I.seed_of("hcx"), device="cuda")
    y = nm.spmv_hybrid(hyb, x)
    f = flags.cpu().numpy().astype(bool)
    yref, A = oracle.hybrid_spmv(bits(W), f, 2, 4, dt, bits(x), keep=keep.cpu().numpy())
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)


def test_hybrid_pack_rejects_wrong_row_count(nm):
    W = I.weight(16, 64, torch.float16, 5).cuda()
    flags = torch.zeros(16, dtype=torch.uint8, device="cuda")
    flags[3] = 1
    with pytest.raises(nm.NmError) as e:
        nm.hybrid_pack(W, flags, 2, 2, 4)
    assert e.value.status == nm.NM_ERR_BAD_MASK


def test_hybrid_full_size_llama_gate(nm):
    """Llama-3.1-8B gate shape (14336 x 4096, 2:4 fp16) with 5% dense rows,
    sampled rows checked."""
    R, K = 14336, 4096
    W = I.weight(R, K, torch.float16, I.seed_of("hfW"), device="cuda")
    x = I.activation_normal(1, K, torch.float16, I.seed_of("hfx"), device="cuda", outlier_frac=0.01)
    loss = nm.hybrid_row_loss(W, 2, 4)
    nd = R // 20
    flags = nm.hybrid_select_rows(loss, nd)
    hyb = nm.hybrid_pack(W, flags, nd, 2, 4)
    y = nm.spmv_hybrid(hyb, x)
    rows = sorted({0, R - 1} | set(np.random.default_rng(6).choice(R, 30, replace=False).tolist()) |
                  set(hyb.rows_dense[:5].cpu().numpy().tolist()))
    f = flags.cpu().numpy().astype(bool)[rows]
    Wr = bits(W[rows])
    want = oracle.hybrid_row_loss(Wr, 2, 4, "fp16")
    assert np.array_equal(loss.cpu().numpy()[rows], want)
    yref, A = oracle.hybrid_spmv(Wr, f, 2, 4, "fp16", bits(x))
    ok, worst, idx = oracle.check(bits(y[:, rows]), yref, A, "fp16")
    assert ok, (worst, idx)
