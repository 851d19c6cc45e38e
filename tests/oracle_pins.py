"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, none of which re-types the oracle's own formulas.

Each ``pin_*`` function raises AssertionError on a violation.  They are run by
``test_oracle_pins.py`` against the real oracle, and by
``test_oracle_mutants.py`` against copies of the oracle with planted mistakes,
to show that each plausible mistake fails at least one pin.

Sources of the facts pinned here:
  * SparseDecoding abstract (humanity-list story page, "Abstract"): an N:M
    sparse matrix-vector product whose kept weights are marked by mask bits
    and whose groups sit at a constant stride in the packed values.
  * bedrocknews arXiv 2610.12327v1 article: N:M keeps a fixed count in every
    small block; the product is a sparse matrix times one vector.
  * IEEE 754 binary16 and bfloat16 field layouts, round-to-nearest-even.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NM_ALL = [(n, m) for m in (4, 8) for n in range(1, m)]


# ---- independent 16-bit codecs (numpy's own float16 / float32 routines) ----

def f16_bits(vals):
    a = np.asarray(vals, np.float64)
    h = a.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), a), "value not exactly representable in fp16"
    return h.view(np.uint16)


def bf16_bits(vals):
    a = np.asarray(vals, np.float64)
    f = a.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), a), "value not exactly representable"
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def to_bits(vals, dtype):
    return f16_bits(vals) if dtype == "fp16" else bf16_bits(vals)


def bits_to_f64(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- golden fixtures -------------------------------------------------------

def load_pack_case(path):
    case = {"W": [], "keep": [], "masks": [], "values": []}
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key in ("W", "keep", "masks", "values"):
                case[key].append(rest)
            elif key == "keep" and rest == ["none"]:
                case["keep"] = None
            else:
                case[key] = rest
    dt = case["dtype"][0]
    n, m = int(case["nm"][0]), int(case["nm"][1])
    R, K = int(case["R"][0]), int(case["K"][0])
    W = to_bits([[float(v) for v in row] for row in case["W"]], dt)
    keep = None
    if case["keep"] and case["keep"][0] != ["none"]:
        keep = np.array([[int(v) for v in row] for row in case["keep"]], np.uint8)
    masks = np.array([[int(v, 16) for v in row] for row in case["masks"]], np.uint8)
    values = to_bits([[float(v) for v in row] for row in case["values"]], dt)
    x = to_bits([[float(v) for v in case["x"]]], dt)
    y = np.array([float(v) for v in case["y"]])
    A = np.array([float(v) for v in case["A"]])
    assert W.shape == (R, K) and masks.shape == (R, K // 8) and values.shape == (R, K * n // m)
    return dict(dtype=dt, n=n, m=m, R=R, K=K, W=W, keep=keep, masks=masks, values=values, x=x, y=y, A=A)


def golden_pack_files():
    return sorted(f for f in os.listdir(GOLDEN) if f.startswith("pack_") and f.endswith(".txt"))


def load_round_cases(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                v, b = line.split()
                out.append((float(v), int(b, 16)))
    return out


def pin_golden_pack(fname):
    c = load_pack_case(os.path.join(GOLDEN, fname))
    vals, masks = oracle.pack(c["W"], c["keep"], c["n"], c["m"], c["dtype"])
    assert np.array_equal(masks, c["masks"]), (fname, masks, c["masks"])
    assert np.array_equal(vals, c["values"]), (fname, vals, c["values"])
    y, A = oracle.spmv(vals, masks, c["K"], c["n"], c["m"], c["dtype"], c["x"])
    assert np.array_equal(y[0], c["y"]), (fname, y, c["y"])
    assert np.array_equal(A[0], c["A"]), (fname, A, c["A"])


def pin_golden_rounding():
    for name, dt in (("round_fp16.txt", "fp16"), ("round_bf16.txt", "bf16")):
        for v, bits in load_round_cases(name):
            got = int(oracle.round_to(np.array([v]), dt)[0])
            assert got == bits, (dt, v, hex(got), hex(bits))


# ---- formats ---------------------------------------------------------------

def pin_decode_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in ("fp16", "bf16"):
        got = oracle.decode(allbits, dt)
        ref = bits_to_f64(allbits, dt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), dt
        assert np.array_equal(got[~nan], ref[~nan]), dt
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), dt


def pin_round_trip_and_midpoints():
    """Every finite 16-bit value rounds to itself; the midpoint of two
    neighbours rounds to the one with an even fraction, and anything strictly
    inside the gap rounds to the nearer neighbour."""
    for dt, inf_bits in (("fp16", 0x7C00), ("bf16", 0x7F80)):
        pos = np.arange(0, inf_bits + 1, dtype=np.uint16)           # +0 .. +inf
        vals = bits_to_f64(pos, dt)
        assert np.all(np.diff(vals) > 0)
        assert np.array_equal(oracle.round_to(vals, dt), pos), dt
        assert np.array_equal(oracle.round_to(-vals, dt), pos | 0x8000), dt
        lo, hi = vals[:-2], vals[1:-1]                                # finite neighbours
        mid = (lo + hi) / 2                                           # exact in double
        even = np.where((pos[:-2] & 1) == 0, pos[:-2], pos[1:-1])
        assert np.array_equal(oracle.round_to(mid, dt), even), dt
        above = np.nextafter(mid, np.inf)
        below = np.nextafter(mid, -np.inf)
        assert np.array_equal(oracle.round_to(above, dt), pos[1:-1]), dt
        assert np.array_equal(oracle.round_to(below, dt), pos[:-2]), dt
        # past the largest finite value: below the overflow midpoint stays finite
        maxf, step = vals[-2], vals[-2] - vals[-3]
        assert int(oracle.round_to(np.array([maxf + step / 2]), dt)[0]) == inf_bits
        assert int(oracle.round_to(np.array([np.nextafter(maxf + step / 2, 0)]), dt)[0]) == inf_bits - 1


def pin_round_matches_libraries(seed=1):
    """numpy rounds double -> binary16 directly, to nearest even; float32 ->
    bfloat16 is the same rule on a narrower input, and numpy's float32 cast
    of a double is exact for float32-representable values."""
    rng = np.random.default_rng(seed)
    e = rng.uniform(-27, 16.5, 200000)
    v = np.ldexp(rng.uniform(1, 2, e.size), np.floor(e).astype(int)) * rng.choice([-1, 1], e.size)
    with np.errstate(over="ignore"):
        ref16 = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round_to(v, "fp16"), ref16)
    # float32 inputs, bf16 rounding by integer arithmetic on the float32 bits
    f = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    ref = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.round_to(f.astype(np.float64), "bf16"), ref)


# ---- pack ------------------------------------------------------------------

def _groups(a, m):
    R, K = a.shape
    return a.reshape(R, K // m, m)


def _unpack_bits(masks, K):
    return np.unpackbits(masks, axis=1, bitorder="little")[:, :K].astype(bool)


def _random_w(rng, R, K, dt, ties):
    if ties:
        w = rng.integers(-3, 4, size=(R, K)).astype(np.float64) * 0.25   # many equal magnitudes
    else:
        w = rng.standard_normal((R, K)) * 0.02
    w = w.astype(np.float16).astype(np.float64) if dt == "fp16" else \
        w.astype(np.float32).astype(np.float64)
    if dt == "bf16":
        u = w.astype(np.float32).view(np.uint32) & 0xFFFF0000
        w = u.view(np.float32).astype(np.float64)
    return to_bits(w, dt)


def check_topn_characterisation(W, vals, masks, n, m, dt):
    """The kept set of every group is the unique set of n columns whose
    magnitudes are not below any dropped magnitude, with ties kept from the
    lowest column; values are the kept words in column order."""
    R, K = W.shape
    kept = _unpack_bits(masks, K)
    kg = _groups(kept, m)
    assert np.all(kg.sum(axis=2) == n), "popcount per group"
    mag = np.abs(bits_to_f64(W, dt))
    mg = _groups(mag, m)
    idx = np.arange(m)
    # a dropped column may never beat a kept one, nor tie with a kept one at a higher index
    for j in range(m):
        for k in range(m):
            bad = kg[:, :, j] & ~kg[:, :, k] & ((mg[:, :, k] > mg[:, :, j]) |
                                               ((mg[:, :, k] == mg[:, :, j]) & (idx[k] < idx[j])))
            assert not bad.any(), f"dropped column {k} should be kept over column {j}"
    Wk = np.where(kept, W, 0).astype(np.uint16)
    assert np.array_equal(vals.reshape(R, -1), W[kept].reshape(R, -1)), "values = kept words in order"
    assert np.array_equal(oracle.expand(vals, masks, K, n, m), Wk), "expand(pack(W)) = W on kept, +0 elsewhere"


def pin_topn(seed=2):
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in NM_ALL:
            for ties in (False, True):
                W = _random_w(rng, 13, 64, dt, ties)
                vals, masks = oracle.pack(W, None, n, m, dt)
                check_topn_characterisation(W, vals, masks, n, m, dt)


def pin_magnitude_order():
    """Reading used by the GPU packer: for non-NaN words, comparing
    (bits & 0x7FFF) as unsigned integers orders them exactly as |w|, and a
    word is NaN iff (bits & 0x7FFF) exceeds the infinity pattern."""
    for dt, inf_bits in (("fp16", 0x7C00), ("bf16", 0x7F80)):
        allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        v = bits_to_f64(allbits, dt)
        assert np.array_equal(np.isnan(v), (allbits & 0x7FFF) > inf_bits)
        code = np.arange(inf_bits + 1, dtype=np.uint16)
        mag_pos = np.abs(bits_to_f64(code, dt))
        mag_neg = np.abs(bits_to_f64(code | 0x8000, dt))
        assert np.array_equal(mag_pos, mag_neg)
        assert np.all(np.diff(mag_pos) > 0)                 # strictly increasing with the code


def pin_all_patterns_bruteforce(seed=3):
    """Every keep pattern of every N:M; the packed product equals the exact
    dense product of W masked by the pattern (math.fsum is correctly rounded),
    within the ascending-order double summation bound."""
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in NM_ALL:
            pats = [c for c in itertools.combinations(range(m), n)]
            G = len(pats)
            K = G * m
            while K % 8:
                K += m
            R, B = 3, 2
            keep = np.zeros((R, K), np.uint8)
            for r in range(R):
                for g in range(K // m):
                    for j in pats[(g + r) % G]:
                        keep[r, g * m + j] = 1
            W = _random_w(rng, R, K, dt, False)
            x = _random_w(rng, B, K, dt, False)
            vals, masks = oracle.pack(W, keep, n, m, dt)
            assert np.array_equal(_unpack_bits(masks, K), keep.astype(bool))
            y, A = oracle.spmv(vals, masks, K, n, m, dt, x)
            wd = bits_to_f64(W, dt) * keep
            xd = bits_to_f64(x, dt)
            for b in range(B):
                for r in range(R):
                    terms = wd[r] * xd[b]
                    exact = math.fsum(terms)
                    absum = math.fsum(np.abs(terms))
                    assert abs(y[b, r] - exact) <= K * 2.0 ** -52 * absum, (dt, n, m, b, r)
                    assert abs(A[b, r] - absum) <= K * 2.0 ** -52 * absum
            yd, Ad = oracle.gemv(np.where(keep, W, 0).astype(np.uint16), dt, x)
            assert np.array_equal(yd, y) and np.array_equal(Ad, A)


def pin_closed_forms():
    for dt in ("fp16", "bf16"):
        for n, m in NM_ALL:
            K = 64
            first_n = np.zeros((2, K), bool)
            first_n.reshape(2, K // m, m)[:, :, :n] = True
            expected_masks = np.packbits(first_n, axis=1, bitorder="little")
            # all-zero W (with -0 mixed in) and constant magnitude with mixed signs
            zeros = np.zeros((2, K), np.uint16)
            zeros[1, 1::3] = 0x8000
            one = to_bits([1.0], dt)[0]
            const = np.full((2, K), one, np.uint16)
            const[:, 1::2] |= 0x8000
            for W in (zeros, const):
                vals, masks = oracle.pack(W, None, n, m, dt)
                assert np.array_equal(masks, expected_masks), (dt, n, m)
            # W = 1, x = 1: y = K*n/m exactly
            K2 = 1024
            Wone = np.full((3, K2), one, np.uint16)
            vals, masks = oracle.pack(Wone, None, n, m, dt)
            y, A = oracle.spmv(vals, masks, K2, n, m, dt, np.full((1, K2), one, np.uint16))
            assert np.all(y == K2 * n // m) and np.all(A == K2 * n // m)


def pin_linearity(seed=4):
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in ((2, 4), (4, 8), (3, 8)):
            R, K = 9, 128
            W = _random_w(rng, R, K, dt, False)
            vals, masks = oracle.pack(W, None, n, m, dt)
            x1 = rng.integers(-8, 9, size=K).astype(np.float64)
            x2 = rng.integers(-8, 9, size=K).astype(np.float64)
            xs = to_bits(np.stack([x1, x2, 2 * x1 + 0.5 * x2]), dt)
            y, A = oracle.spmv(vals, masks, K, n, m, dt, xs)
            lhs = y[2]
            rhs = 2 * y[0] + 0.5 * y[1]
            bound = 4 * K * 2.0 ** -52 * (2 * A[0] + 0.5 * A[1] + A[2])
            assert np.all(np.abs(lhs - rhs) <= bound), (dt, n, m)


def pin_one_hot(seed=5):
    """x = e_j picks column j of the pruned matrix exactly (subnormal weights
    included)."""
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in ((2, 4), (4, 8), (1, 8)):
            R, K = 5, 32
            W = _random_w(rng, R, K, dt, False)
            W[:, ::5] = rng.integers(1, 0x7F, size=W[:, ::5].shape).astype(np.uint16)   # subnormals
            W[0, 3] |= 0x8000
            vals, masks = oracle.pack(W, None, n, m, dt)
            Wt = np.where(_unpack_bits(masks, K), bits_to_f64(W, dt), 0.0)
            one = to_bits([1.0], dt)[0]
            x = np.zeros((K, K), np.uint16)
            x[np.arange(K), np.arange(K)] = one
            y, _ = oracle.spmv(vals, masks, K, n, m, dt, x)
            assert np.array_equal(y, Wt.T), (dt, n, m)


def pin_integer_exact(seed=6):
    """w in {-8..8}/16 and x in {-8..8}: the sum is an exact rational; the
    oracle's double sum must equal it and its rounding must be the
    correctly-rounded 16-bit value of that rational."""
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in ((2, 4), (4, 8), (3, 4)):
            R, K, B = 6, 256, 3
            wi = rng.integers(-8, 9, size=(R, K))
            xi = rng.integers(-8, 9, size=(B, K))
            W = to_bits(wi / 16.0, dt)
            x = to_bits(xi.astype(np.float64), dt)
            vals, masks = oracle.pack(W, None, n, m, dt)
            kept = _unpack_bits(masks, K)
            y, _ = oracle.spmv(vals, masks, K, n, m, dt, x)
            for b in range(B):
                for r in range(R):
                    exact = Fraction(int(np.sum(wi[r] * kept[r] * xi[b])), 16)
                    assert Fraction(y[b, r]) == exact, (dt, n, m, b, r)


def pin_errors():
    W = to_bits(np.ones((2, 16)), "fp16")
    bad_keep = np.zeros((2, 16), np.uint8)
    bad_keep[:, ::4] = 1                                         # one per group, not two
    for call in (lambda: oracle.pack(W, bad_keep, 2, 4, "fp16"),):
        try:
            call()
        except oracle.OracleError as e:
            assert e.status == oracle.BAD_MASK
        else:
            raise AssertionError("bad keep-mask accepted")
    Wn = W.copy()
    Wn[1, 5] = 0x7E00
    try:
        oracle.pack(Wn, None, 2, 4, "fp16")
    except oracle.OracleError as e:
        assert e.status == oracle.NONFINITE
    else:
        raise AssertionError("NaN accepted in top-N mode")
    # keep-mask mode copies NaN words verbatim
    good_keep = np.zeros((2, 16), np.uint8)
    good_keep[:, 0::4] = 1
    good_keep[:, 1::4] = 1
    vals, _ = oracle.pack(Wn, good_keep, 2, 4, "fp16")
    assert vals[1, 3] == 0x7E00                                 # column 5 = group 1, second kept
    for (R, K, n, m) in ((2, 12, 2, 4), (2, 16, 2, 3), (2, 16, 4, 4), (2, 16, 0, 4), (2, 16, 8, 8)):
        try:
            oracle.pack(np.ones((R, K), np.uint16), None, n, m, "fp16")
        except (oracle.OracleError, ValueError) as e:
            assert not isinstance(e, oracle.OracleError) or e.status == oracle.BAD_SHAPE
        else:
            raise AssertionError(f"shape {(R, K, n, m)} accepted")


def pin_silu():
    """SiLU against closed forms: SiLU(0) = 0; sigmoid(ln 3) = 3/4, so
    SiLU(+-ln 3) = 3/4 ln 3 and -1/4 ln 3; SiLU(t) - SiLU(-t) = t; SiLU(t) -> t
    for large t and -> 0 for very negative t; the minimum sits at
    t* = -1 - W(1/e) (Lambert W) with value t* + 1 (there 1 + t (1 - sigmoid) = 0,
    so sigmoid = 1 + 1/t and t sigmoid = t + 1)."""
    from scipy.special import lambertw
    ln3 = math.log(3.0)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(ln3) - 0.75 * ln3) <= 4e-16
    assert abs(oracle.silu(-ln3) + 0.25 * ln3) <= 4e-16
    for t in np.concatenate([np.linspace(0.01, 30.0, 97), [1e-6, 1e-3, 2.5, 7.0]]):
        assert abs(oracle.silu(t) - oracle.silu(-t) - t) <= 1e-15 * max(1.0, t)
    assert oracle.silu(50.0) == 50.0
    assert oracle.silu(-800.0) == 0.0
    tstar = -1.0 - float(lambertw(math.exp(-1.0)).real)
    assert abs(oracle.silu(tstar) - (tstar + 1.0)) <= 1e-15
    grid = np.linspace(-4.0, 1.0, 5001)
    vals = np.array([oracle.silu(t) for t in grid])
    assert abs(grid[int(np.argmin(vals))] - tstar) <= 1e-3
    assert vals.min() >= tstar + 1.0 - 1e-15


def pin_swiglu():
    """h = SiLU(g) * u elementwise: known values, u = 1 gives SiLU itself, and
    the roles of g and u are not symmetric (swapping them changes h)."""
    ln3 = math.log(3.0)
    h = oracle.swiglu(np.array([ln3, 0.0, -ln3, 2.0]), np.array([2.0, 5.0, 4.0, -1.0]))
    want = np.array([1.5 * ln3, 0.0, -ln3, -2.0 / (1.0 + math.exp(-2.0))])
    assert np.all(np.abs(h - want) <= 4e-16 * np.maximum(1.0, np.abs(want)))
    g = np.linspace(-6.0, 6.0, 49)
    assert np.array_equal(oracle.swiglu(g, np.ones_like(g)), np.array([oracle.silu(t) for t in g]))
    assert oracle.swiglu(np.array([3.0]), np.array([-2.0]))[0] != oracle.swiglu(np.array([-2.0]), np.array([3.0]))[0]


def _bitmap_to_keep(masks, K):
    """1-bit-per-column bitmap [R][K/8] -> keep bytes [R][K]."""
    return np.unpackbits(np.ascontiguousarray(masks, np.uint8), axis=1, bitorder="little")[:, :K]


def pin_calib_accumulate(seed=7):
    """H = sum over decode rows of x x^T against independent routes: numpy's
    matmul of the selected rows (integer-valued, so exact), one-hot rows
    (H diagonal), rank-one rows c_t (1..K) (H_ij = sum c_t^2 i j), the decode
    mask (all-zero mask gives 0; None equals all ones), accumulation across
    calls, symmetry and the trace."""
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        T, K = 9, 16
        Xv = rng.integers(-6, 7, size=(T, K)).astype(np.float64)
        X = to_bits(Xv, dt)
        d = (rng.random(T) < 0.6).astype(np.uint8)
        d[0], d[1] = 0, 1
        H, A = oracle.calib_accumulate(X, dt, decode=d)
        Xd = Xv[d != 0]
        assert np.array_equal(H, Xd.T @ Xd)
        assert np.array_equal(A, np.abs(Xd).T @ np.abs(Xd))
        assert np.array_equal(H, H.T) and np.trace(H) == float((Xd ** 2).sum())
        H0, _ = oracle.calib_accumulate(X, dt, decode=np.zeros(T, np.uint8))
        assert not H0.any()
        Hn, _ = oracle.calib_accumulate(X, dt)
        Ho, _ = oracle.calib_accumulate(X, dt, decode=np.ones(T, np.uint8))
        assert np.array_equal(Hn, Ho) and np.array_equal(Hn, Xv.T @ Xv)
        # accumulation: two calls equal one call over both row sets
        H1, A1 = oracle.calib_accumulate(X[:4], dt)
        H2, _ = oracle.calib_accumulate(X[4:], dt, H=H1, A=A1)
        assert np.array_equal(H2, Hn)
        # one-hot rows: diagonal H
        idx = rng.integers(0, K, size=T)
        vals = rng.integers(1, 5, size=T).astype(np.float64)
        Xo = np.zeros((T, K))
        Xo[np.arange(T), idx] = vals
        Ho, _ = oracle.calib_accumulate(to_bits(Xo, dt), dt)
        want = np.zeros((K, K))
        for t in range(T):
            want[idx[t], idx[t]] += vals[t] ** 2
        assert np.array_equal(Ho, want)
        # rank-one rows c_t * (1, 2, ..., K)
        c = np.array([1.0, -2.0, 0.5])
        Xr = np.outer(c, np.arange(1, K + 1))
        Hr, _ = oracle.calib_accumulate(to_bits(Xr, dt), dt)
        assert np.array_equal(Hr, (c ** 2).sum() * np.outer(np.arange(1, K + 1), np.arange(1, K + 1)))


def _keep_brute(Wv, h, n, m):
    """Top-n per m-group by exact rational saliency w^2 h (finite inputs),
    lower column first on ties, by sorting."""
    R, K = Wv.shape
    keep = np.zeros((R, K), np.uint8)
    for r in range(R):
        for g0 in range(0, K, m):
            sal = [Fraction(Wv[r, g0 + j]) ** 2 * Fraction(float(h[g0 + j])) for j in range(m)]
            order = sorted(range(m), key=lambda j: (-sal[j], j))
            for j in order[:n]:
                keep[r, g0 + j] = 1
    return keep


def pin_calib_keep(seed=8):
    """Saliency keep-mask: equals the magnitude rule when h is constant (a
    reduction to the pinned top-n by |w|), the top-n of h when |w| is
    constant, exact-rational brute force on random inputs, and a NaN saliency
    ranks below every number, -inf included."""
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in ((2, 4), (4, 8), (1, 4), (3, 8)):
            R, K = 6, 32
            Wv = np.round(rng.normal(0, 1, (R, K)) * 8) / 8           # many equal magnitudes
            W = to_bits(Wv, dt)
            Wv = bits_to_f64(W, dt)
            # constant h: the magnitude rule
            _, masks = oracle.pack(W, None, n, m, dt)
            assert np.array_equal(oracle.calib_keep(W, np.full(K, 3.0), n, m, dt), _bitmap_to_keep(masks, K))
            # constant |w|: the largest h, lower column on ties
            ones = to_bits(np.where(rng.random((R, K)) < 0.5, -1.0, 1.0), dt)
            h = rng.integers(0, 4, size=K).astype(np.float32)
            got = oracle.calib_keep(ones, h, n, m, dt)
            want = np.zeros((R, K), np.uint8)
            for g0 in range(0, K, m):
                order = sorted(range(m), key=lambda j: (-h[g0 + j], j))
                want[:, [g0 + j for j in order[:n]]] = 1
            assert np.array_equal(got, want)
            # brute force with exact rationals
            h = (rng.random(K) * 4).astype(np.float32)
            h[rng.random(K) < 0.2] = 0.0
            assert np.array_equal(oracle.calib_keep(W, h, n, m, dt), _keep_brute(Wv, h.astype(np.float64), n, m))
    # NaN saliency ranks below everything (fp16 0x7E00 = NaN)
    W = np.array([[0x7E00, 0x3C00, 0x7E00, 0x0000, 0x3C00, 0x4000, 0x3C00, 0x4000]], np.uint16)  # NaN 1 NaN 0 | 1 2 1 2
    keep = oracle.calib_keep(W, np.ones(8, np.float32), 2, 4, "fp16")
    assert keep.tolist() == [[0, 1, 0, 1, 0, 1, 0, 1]]
    keep = oracle.calib_keep(W, np.ones(8, np.float32), 3, 4, "fp16")
    assert keep.tolist() == [[1, 1, 0, 1, 1, 1, 0, 1]]
    # ... negative saliencies included: NaN, -2, -3, -1 keep columns 3 and 1 (then a group of equal ones)
    W = np.array([[0x7E00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00]], np.uint16)
    keep = oracle.calib_keep(W, np.array([1.0, -2.0, -3.0, -1.0, 1.0, 1.0, 1.0, 1.0], np.float32), 2, 4, "fp16")
    assert keep.tolist() == [[0, 1, 0, 1, 1, 1, 0, 0]]
    # ... and below -inf: saliencies NaN, -inf, 2, 3 | -inf, NaN, 2, 3 keep -inf over NaN in either order
    inf = float("inf")
    W = np.array([[0x7E00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x7E00, 0x3C00, 0x3C00]], np.uint16)
    h = np.array([1.0, -inf, 2.0, 3.0, -inf, 1.0, 2.0, 3.0], np.float32)
    assert oracle.calib_keep(W, h, 3, 4, "fp16").tolist() == [[0, 1, 1, 1, 1, 0, 1, 1]]
    assert oracle.calib_keep(W, h, 1, 4, "fp16").tolist() == [[0, 0, 0, 1, 0, 0, 0, 1]]
    # a zero weight under h = -inf gives 0 * -inf = NaN, which also ranks last
    W = np.array([[0x0000, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x0000]], np.uint16)
    h = np.array([-inf, -inf, 1.0, 1.0, 1.0, 1.0, -inf, -inf], np.float32)
    assert oracle.calib_keep(W, h, 3, 4, "fp16").tolist() == [[0, 1, 1, 1, 1, 1, 1, 0]]


def pin_hybrid(seed=9):
    """Hybrid rows: the row loss against exact rationals over the pruned
    columns (taken from the pinned packer's bitmap), in top-n and keep-mask
    modes; scaling h by 4 scales the loss by 4 exactly; the row choice against
    a sort (loss descending, row ascending), with n_dense = 0 and = R, ties
    and a NaN loss; and the hybrid product reduces to the sparse product with
    no dense rows and to the dense product with all rows dense."""
    rng = np.random.default_rng(seed)
    for dt in ("fp16", "bf16"):
        for n, m in ((2, 4), (4, 8), (1, 4)):
            R, K = 9, 32
            Wv = np.round(rng.normal(0, 1, (R, K)) * 8) / 8
            W = to_bits(Wv, dt)
            Wv = bits_to_f64(W, dt)
            h = (rng.random(K) * 4).astype(np.float32)
            rand_keep = np.zeros((R, K), np.uint8)
            for r in range(R):
                for g0 in range(0, K, m):
                    rand_keep[r, g0 + rng.choice(m, size=n, replace=False)] = 1
            for keep in (None, rand_keep):
                loss = oracle.hybrid_row_loss(W, n, m, dt, keep=keep, h=h)
                kept = _bitmap_to_keep(oracle.pack(W, keep, n, m, dt)[1], K).astype(bool)
                for r in range(R):
                    exact = sum(Fraction(Wv[r, c]) ** 2 * Fraction(float(h[c])) for c in range(K) if not kept[r, c])
                    assert abs(Fraction(loss[r]) - exact) <= Fraction(1, 10 ** 12) * (1 + abs(exact))
                assert np.array_equal(oracle.hybrid_row_loss(W, n, m, dt, keep=keep, h=4 * h), 4 * loss)
            loss1 = oracle.hybrid_row_loss(W, n, m, dt)
            for r in range(R):
                _, mk = oracle.pack(W[r:r + 1], None, n, m, dt)
                kept = _bitmap_to_keep(mk, K)[0].astype(bool)
                assert loss1[r] == math.fsum(Wv[r, c] ** 2 for c in range(K) if not kept[c]) or \
                    abs(loss1[r] - math.fsum(Wv[r, c] ** 2 for c in range(K) if not kept[c])) <= 1e-12 * loss1[r]
    # NaN ranks below every number, negative and -inf included; NaNs tie among
    # themselves (lower row first among equals, as for numbers)
    nan, inf = float("nan"), float("inf")
    for loss in (np.array([3.0, 1.0, 3.0, nan, 0.0, 7.0, 1.0]),
                 np.array([-5.0, nan, -0.5, 2.0, -inf, -5.0, nan]),
                 np.array([nan, -inf, nan, -inf, inf, nan, -0.0, 0.0])):
        for nd in range(len(loss) + 1):
            order = sorted(range(len(loss)), key=lambda r: (math.isnan(loss[r]), 0.0 if math.isnan(loss[r]) else -loss[r], r))
            want = np.zeros(len(loss), np.uint8)
            want[order[:nd]] = 1
            assert np.array_equal(oracle.hybrid_select(loss, nd), want)
    assert list(oracle.hybrid_select(np.array([nan, -2.0]), 1)) == [0, 1]
    assert list(oracle.hybrid_select(np.array([nan, -inf]), 1)) == [0, 1]
    assert list(oracle.hybrid_select(np.array([-inf, nan]), 1)) == [1, 0]
    assert list(oracle.hybrid_select(np.array([nan, nan, -inf]), 2)) == [1, 0, 1]
    # the product reduces to the plain ones
    R, K = 6, 64
    W = to_bits(np.round(rng.normal(0, 1, (R, K)) * 16) / 16, "fp16")
    x = to_bits(np.round(rng.normal(0, 1, (2, K)) * 16) / 16, "fp16")
    v, mk = oracle.pack(W, None, 2, 4, "fp16")
    ys, _ = oracle.spmv(v, mk, K, 2, 4, "fp16", x)
    yd, _ = oracle.gemv(W, "fp16", x)
    assert np.array_equal(oracle.hybrid_spmv(W, np.zeros(R, np.uint8), 2, 4, "fp16", x)[0], ys)
    assert np.array_equal(oracle.hybrid_spmv(W, np.ones(R, np.uint8), 2, 4, "fp16", x)[0], yd)
    f = np.array([1, 0, 0, 1, 0, 1], np.uint8)
    yh = oracle.hybrid_spmv(W, f, 2, 4, "fp16", x)[0]
    assert np.array_equal(yh[:, f == 1], yd[:, f == 1]) and np.array_equal(yh[:, f == 0], ys[:, f == 0])


ALL_PINS = [
    pin_golden_rounding,
    pin_decode_exhaustive,
    pin_round_trip_and_midpoints,
    pin_round_matches_libraries,
    pin_topn,
    pin_all_patterns_bruteforce,
    pin_closed_forms,
    pin_linearity,
    pin_one_hot,
    pin_integer_exact,
    pin_errors,
    pin_silu,
    pin_swiglu,
    pin_calib_accumulate,
    pin_calib_keep,
    pin_hybrid,
] + [(lambda f=f: pin_golden_pack(f)) for f in golden_pack_files()]
