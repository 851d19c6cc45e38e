"""GPU parity of decoding-aware calibration through the C ABI:
``nm_calib_accumulate`` (H += X_d^T X_d on the matrix cores) against the
oracle's double sums, and ``nm_calib_keep_mask`` (top-N of w^2 H_jj per group)
bit for bit against the oracle given the same fp32 diagonal; then the whole
offline flow, calibration -> keep-mask -> nm_pack -> nm_spmv."""
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


def decode_flags(T, seed, frac=0.7):
    g = np.random.default_rng(seed)
    d = (g.random(T) < frac).astype(np.uint8)
    if T:
        d[0] = 0                                   # a prefill row first, as in a real trace
    return d


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("T,K", [(1, 8), (37, 136), (100, 264), (70, 128)])
@pytest.mark.parametrize("masked", [False, True])
def test_calib_accumulate(nm, dt, T, K, masked):
    X = I.activation_normal(T, K, TD[dt], I.seed_of("calX", T, K, dt))
    d = decode_flags(T, I.seed_of("cald", T)) if masked else None
    H = nm.calib_accumulate(X.cuda(), None if d is None else torch.from_numpy(d).cuda())
    Href, A = oracle.calib_accumulate(bits(X), dt, decode=d)
    ok, worst, idx = oracle.check_calib(H.cpu().numpy(), Href, A)
    assert ok, (worst, idx)
    # a second call adds to H (here: the same rows again, unmasked)
    H0 = H.cpu().numpy().astype(np.float64)
    nm.calib_accumulate(X.cuda(), None, H=H)
    Href2, A2 = oracle.calib_accumulate(bits(X), dt, H=Href, A=A)
    ok, worst, idx = oracle.check_calib(H.cpu().numpy(), Href2, A2, H0=H0)
    assert ok, (worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("T,K", [(150, 392), (300, 520), (64, 256), (129, 136)])
def test_calib_accumulate_onto_unsymmetric_h(nm, dt, T, K):
    """H starts as an arbitrary (unsymmetric) matrix: every entry, on both
    sides of the diagonal, must receive its own H0 plus the sums.  Token
    counts give an odd number of 64-row steps, a partial last step and an
    exact one; K gives ragged edge tiles and several off-diagonal tiles."""
    X = I.activation_normal(T, K, TD[dt], I.seed_of("calU", T, K, dt))
    d = decode_flags(T, I.seed_of("caldU", T))
    H0 = torch.from_numpy(np.random.default_rng(T + K).standard_normal((K, K)).astype(np.float32))
    H = H0.cuda()
    nm.calib_accumulate(X.cuda(), torch.from_numpy(d).cuda(), H=H)
    Href, A = oracle.calib_accumulate(bits(X), dt, decode=d, H=H0.numpy().astype(np.float64))
    ok, worst, idx = oracle.check_calib(H.cpu().numpy(), Href, A, H0=H0.numpy())
    assert ok, (worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_calib_accumulate_nonfinite_prefill_rows_excluded(nm, dt):
    """Prefill rows holding Inf and NaN do not reach H: rows flagged as
    prefill contribute nothing, not 0 * Inf.  T = 100 puts flagged rows in
    every 32-token stage, the partial last one included."""
    T, K = 100, 264
    X = I.activation_normal(T, K, TD[dt], I.seed_of("calNF", dt))
    d = np.ones(T, np.uint8)
    bad = [0, 5, 31, 32, 63, 70, 99]
    d[bad] = 0
    Xb = X.clone()
    Xb[bad[0::2], :] = float("inf")
    Xb[bad[1::2], 7] = float("nan")
    Xb[bad[1::2], 100] = -float("inf")
    H = nm.calib_accumulate(Xb.cuda(), torch.from_numpy(d).cuda()).cpu().numpy()
    assert np.isfinite(H).all()
    Href, A = oracle.calib_accumulate(bits(X), dt, decode=d)
    ok, worst, idx = oracle.check_calib(H, Href, A)
    assert ok, (worst, idx)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_calib_accumulate_integer_exact(nm, dt):
    """Integer-valued rows: every partial sum is an integer below 2^24, so H
    must equal the exact sums in any order."""
    T, K = 64, 264
    X = I.integer_valued(T, K, TD[dt], I.seed_of("calI", dt), lo=-3, hi=3)
    d = decode_flags(T, 11)
    H = nm.calib_accumulate(X.cuda(), torch.from_numpy(d).cuda())
    Href, _ = oracle.calib_accumulate(bits(X), dt, decode=d)
    assert np.array_equal(H.cpu().numpy().astype(np.float64), Href)


def test_calib_accumulate_one_hot_rows(nm):
    """Rows with a single nonzero entry give a diagonal H: any slip in the
    matrix-core result layout shows up as off-diagonal or misplaced values."""
    T, K = 300, 392
    g = np.random.default_rng(12)
    cols = g.integers(0, K, size=T)
    vals = g.integers(1, 9, size=T).astype(np.float32)
    Xf = np.zeros((T, K), np.float32)
    Xf[np.arange(T), cols] = vals
    X = torch.from_numpy(Xf).to(torch.float16)
    H = nm.calib_accumulate(X.cuda()).cpu().numpy()
    want = np.zeros((K, K), np.float32)
    for t in range(T):
        want[cols[t], cols[t]] += vals[t] ** 2
    assert np.array_equal(H, want)


def test_calib_accumulate_full_size_sampled(nm):
    """Llama-3.1-8B hidden size (K = 4096), 512 rows with a prefill block:
    entries H[S][S] for a sampled column set S against the oracle on X[:, S]
    (the same sums restricted to those columns)."""
    T, K = 512, 4096
    X = I.activation_normal(T, K, torch.bfloat16, I.seed_of("calF"), device="cuda", outlier_frac=0.01)
    d = np.ones(T, np.uint8)
    d[:96] = 0                                     # the prompt's prefill rows
    H = nm.calib_accumulate(X, torch.from_numpy(d).cuda())
    S = np.sort(np.random.default_rng(13).choice(K, size=96, replace=False))
    S[0], S[-1] = 0, K - 1
    Href, A = oracle.calib_accumulate(bits(X)[:, S], "bf16", decode=d)
    Hs = H.cpu().numpy()[np.ix_(S, S)]
    ok, worst, idx = oracle.check_calib(Hs, Href, A)
    assert ok, (worst, idx)


def test_calib_accumulate_largest_k(nm):
    """K = 65536, the largest the call accepts: a 16 GB H, 131328 upper-
    triangle tiles; entries H[S][S] for sampled columns S (both sides of the
    diagonal, the last tile included) against the oracle on X[:, S]."""
    T, K = 40, 65536
    X = I.activation_normal(T, K, torch.bfloat16, I.seed_of("calK"), device="cuda")
    d = np.ones(T, np.uint8)
    d[:3] = 0
    H = torch.zeros((K, K), dtype=torch.float32, device="cuda")
    H[0, K - 1] = 2.0                              # prior contents, off the diagonal
    H[K - 1, 0] = -3.0
    nm.calib_accumulate(X, torch.from_numpy(d).cuda(), H=H)
    S = np.sort(np.random.default_rng(31).choice(K, size=48, replace=False))
    S[0], S[-1] = 0, K - 1
    Hs = H[torch.from_numpy(S).cuda()][:, torch.from_numpy(S).cuda()].cpu().numpy()
    del H
    torch.cuda.empty_cache()
    H0 = np.zeros((len(S), len(S)), np.float64)
    H0[0, -1], H0[-1, 0] = 2.0, -3.0
    Href, A = oracle.calib_accumulate(bits(X)[:, S], "bf16", decode=d, H=H0)
    ok, worst, idx = oracle.check_calib(Hs, Href, A, H0=H0)
    assert ok, (worst, idx)


def test_calib_accumulate_empty(nm):
    H = torch.full((16, 16), 3.0, device="cuda")
    nm.calib_accumulate(torch.empty((0, 16), dtype=torch.float16, device="cuda"), None, H=H)
    assert torch.all(H == 3.0)
    d = torch.zeros(5, dtype=torch.uint8, device="cuda")            # all prefill: nothing enters H
    nm.calib_accumulate(torch.ones((5, 16), dtype=torch.float16, device="cuda"), d, H=H)
    assert torch.all(H == 3.0)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (1, 4), (3, 8)])
def test_calib_keep_mask_bitexact(nm, dt, n, m):
    R, K = 37, 264
    W = I.weight(R, K, TD[dt], I.seed_of("ckW", dt, n, m))
    W = (torch.round(W.float() / 0.004) * 0.004).to(TD[dt])         # many equal |w| -> saliency ties
    g = np.random.default_rng(I.seed_of("ckh", dt, n, m))
    h = g.integers(0, 5, size=K).astype(np.float32)                # equal h values -> more ties
    h[:3] = [0.0, 1e-40, 3.0e38]                                   # zero, an fp32 subnormal, a huge value
    keep = nm.calib_keep_mask(W.cuda(), torch.from_numpy(h).cuda(), n, m).cpu().numpy()
    want = oracle.calib_keep(bits(W), h, n, m, dt)
    assert np.array_equal(keep, want)
    assert np.all(keep.reshape(R, K // m, m).sum(-1) == n)


def test_calib_keep_mask_nan_and_full_h(nm):
    """NaN weights rank lowest; a full [K][K] H is read on its diagonal."""
    R, K = 5, 64
    W = I.weight(R, K, torch.float16, I.seed_of("ckN"))
    W[0, 0] = float("nan")
    W[1, 4:8] = float("nan")
    Hfull = torch.from_numpy(np.random.default_rng(14).random((K, K)).astype(np.float32))
    keep = nm.calib_keep_mask(W.cuda(), Hfull.cuda(), 2, 4).cpu().numpy()
    want = oracle.calib_keep(bits(W), np.diag(Hfull.numpy()).copy(), 2, 4, "fp16")
    assert np.array_equal(keep, want)
    assert keep[0, 0] == 0 and keep[1, 4:8].tolist() == [1, 1, 0, 0]


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_calib_keep_mask_negative_saliency_and_nan(nm, n, m):
    """A caller's h may hold negative values: NaN saliencies still rank below
    every number, negative ones included."""
    R, K = 6, 64
    W = I.weight(R, K, torch.bfloat16, I.seed_of("ckNeg", n, m))
    W[0, 0] = float("nan")
    W[2, 8:12] = float("nan")
    h = (np.random.default_rng(17).random(K) * 4 - 3).astype(np.float32)   # mostly negative
    keep = nm.calib_keep_mask(W.cuda(), torch.from_numpy(h).cuda(), n, m).cpu().numpy()
    assert np.array_equal(keep, oracle.calib_keep(bits(W), h, n, m, "bf16"))
    assert keep[0, 0] == 0


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_calib_keep_mask_nan_below_minus_inf(nm, dt):
    """A NaN saliency ranks below -inf: groups holding both (NaN first or
    -inf first, and 0 * -inf = NaN) keep the -inf column before the NaN one."""
    tdt = TD[dt]
    inf, nan = float("inf"), float("nan")
    W = torch.tensor([[nan, 1.0, 1.0, 1.0, 1.0, nan, 1.0, 1.0, 0.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 0.0]], dtype=tdt)
    h = np.array([1.0, -inf, 2.0, 3.0, -inf, 1.0, 2.0, 3.0, -inf, -inf, 1.0, 1.0, 1.0, 1.0, -inf, -inf], np.float32)
    for n in (1, 2, 3):
        keep = nm.calib_keep_mask(W.cuda(), torch.from_numpy(h).cuda(), n, 4).cpu().numpy()
        assert np.array_equal(keep, oracle.calib_keep(bits(W), h, n, 4, dt)), n
    keep = nm.calib_keep_mask(W.cuda(), torch.from_numpy(h).cuda(), 3, 4).cpu().numpy()
    assert keep[0].tolist() == [0, 1, 1, 1, 1, 0, 1, 1, 0, 1, 1, 1, 1, 1, 1, 0]


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_calibrated_pack_and_spmv(nm, dt):
    """The offline flow end to end on a Llama-3.1-8B-shaped layer slice:
    decode-step activations -> H -> keep-mask -> nm_pack -> nm_spmv, each
    stage checked against the oracle (the keep-mask from the GPU's own fp32
    diagonal, so that both sides decide on the same numbers)."""
    R, K, T = 256, 4096, 200
    tdt = TD[dt]
    W = I.weight(R, K, tdt, I.seed_of("e2eW", dt))
    X = I.activation_normal(T, K, tdt, I.seed_of("e2eX", dt), outlier_frac=0.01)
    d = decode_flags(T, 15)
    H = nm.calib_accumulate(X.cuda(), torch.from_numpy(d).cuda())
    hdiag = torch.diagonal(H).contiguous().cpu().numpy()
    keep = nm.calib_keep_mask(W.cuda(), H, 2, 4)
    assert np.array_equal(keep.cpu().numpy(), oracle.calib_keep(bits(W), hdiag, 2, 4, dt))
    v, mk = nm.pack(W.cuda(), keep, 2, 4)
    ov, om = oracle.pack(bits(W), keep.cpu().numpy(), 2, 4, dt)
    assert np.array_equal(bits(v), ov) and np.array_equal(mk.cpu().numpy(), om)
    x = I.activation_normal(1, K, tdt, I.seed_of("e2ex", dt))
    y = nm.spmv(v, mk, x.cuda(), 2, 4)
    yref, A = oracle.spmv(ov, om, K, 2, 4, dt, bits(x))
    ok, worst, idx = oracle.check(bits(y), yref, A, dt)
    assert ok, (worst, idx)
    # the calibrated mask differs from plain magnitude pruning where activations differ in scale
    _, mag = oracle.pack(bits(W), None, 2, 4, dt)
    assert not np.array_equal(om, mag)
