"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin is a small check function; the tests run it on the oracle as written
and, for the pins that guard arithmetic, on a copy of the oracle with a
planted mistake (a dropped term, a wrong sign, a swapped bit order...), which
the pin must catch.
"""

import json
import os

import numpy as np
import pytest

from oracle import accounting, encode, gemv, pack
from synth import WORKLOADS, make_weights, make_x, outlier_count

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# Pin 1: the CSR worked example printed on the SpQR page
# ---------------------------------------------------------------------------
def _spqr_example_matrix(seed=0):
    g = _golden("spqr_csr_example.json")
    M, K = g["shape"]
    rng = np.random.default_rng(seed)
    W = rng.uniform(-g["bulk_abs_max"], g["bulk_abs_max"], size=(M, K))
    for i, j, v in g["outliers"]:
        W[i, j] = v
    return W.astype(np.float16), g


def check_csr_example(bits, fmt, seed=0):
    W, g = _spqr_example_matrix(seed)
    x = np.ones(W.shape[1])
    enc = encode.encode(W, bits, fmt, len(g["outliers"]), 16, sens=x)
    ok = (list(enc["col_idx"]) == g["col_idx"]
          and list(enc["row_ptr"]) == g["row_ptr"]
          and [hex(v) for v in _f16bits(enc["values"])] == g["values_fp16_bits"]
          and list(enc["values"].astype(np.float64)) == g["values_decimal"])
    D = gemv.decode(enc)
    holes_zero = all(D[i, j] == 0.0 for i, j, _ in g["outliers"])
    return ok and holes_zero


@pytest.mark.parametrize("bits,fmt", [(3, "uniform"), (4, "uniform"), (3, "lut"), (4, "lut")])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_csr_worked_example(bits, fmt, seed):
    assert check_csr_example(bits, fmt, seed)


def test_csr_worked_example_catches_sign_flip(monkeypatch):
    orig = encode.build_csr

    def flipped(W16, hole, D):
        rp, ci, v = orig(W16, hole, D)
        return rp, ci, (-v.astype(np.float64)).astype(np.float16)
    monkeypatch.setattr(encode, "build_csr", flipped)
    assert not check_csr_example(3, "uniform")


def test_csr_worked_example_catches_column_major_order(monkeypatch):
    orig = encode.build_csr

    def colmajor(W16, hole, D):
        rp, ci, v = orig(W16, hole, D)
        c, r = np.nonzero(hole.T)          # column-major traversal
        return rp, c.astype(np.int32), v
    monkeypatch.setattr(encode, "build_csr", colmajor)
    assert not check_csr_example(3, "uniform")


# ---------------------------------------------------------------------------
# Pin 2: W_dense + W_sparse reproduces every outlier exactly
# ---------------------------------------------------------------------------
SMALL = {
    "tiny_u4": (None, None),
    "attn7b_u3": (48, 4096),
    "mlp7b_lut3": (24, 4096),
    "mlp70b_lut4": (16, 8192),
    "block7b_u3": (64, 2048),
}


def _small_encoding(name):
    wl = WORKLOADS[name]
    M, K = SMALL[name]
    W, planted = make_weights(wl, 0, M, K)
    M, K = W.shape
    x = make_x(wl, max(wl.batches), K, 0, M)
    enc = encode.encode(W, wl.bits, wl.fmt, outlier_count(wl, M, K), wl.group or 16,
                        sens=x[0].astype(np.float64) ** 2)
    return wl, W, planted, x, enc


_CACHE = {}


def small(name):
    if name not in _CACHE:
        _CACHE[name] = _small_encoding(name)
    return _CACHE[name]


def check_exact_outliers(W, enc):
    D = gemv.decode(enc)
    r, c = np.nonzero(enc["mask"])
    recon = D[r, c] + enc["values"].astype(np.float64)
    return bool(np.array_equal(recon, W.astype(np.float64)[r, c]))


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_plus_sparse_exact_at_outliers(name):
    wl, W, planted, x, enc = small(name)
    assert np.array_equal(enc["mask"], planted)
    assert check_exact_outliers(W, enc)
    assert enc["row_ptr"][-1] == planted.sum()


def test_exactness_catches_nonzero_hole(monkeypatch):
    wl, W, planted, x, enc = small("tiny_u4")
    orig = encode.quant_uniform

    def bad(W16, hole, bits, group):
        q, s, z = orig(W16, hole, bits, group)
        q = q.copy()
        q[hole] = np.minimum(q[hole] + 1, (1 << bits) - 1)
        return q, s, z
    monkeypatch.setattr(encode, "quant_uniform", bad)
    enc2 = encode.encode(W, 4, "uniform", outlier_count(wl, *W.shape), 16)
    assert not check_exact_outliers(W, enc2)


# ---------------------------------------------------------------------------
# Pin 3: brute-force GEMV straight from the packed bytes (pure Python loops)
# ---------------------------------------------------------------------------
def brute_force_y(enc, X16):
    """Triple loop over the canonical arrays; bits extracted one by one."""
    M, K, b = enc["M"], enc["K"], enc["bits"]
    packed = np.asarray(enc["codes_packed"])
    rp, ci, va = enc["row_ptr"], enc["col_idx"], enc["values"]
    Y = []
    for xrow in np.asarray(X16):
        x = [float(v) for v in xrow]
        y = []
        for i in range(M):
            row = [int(v) for v in packed[i]]
            acc = 0.0
            for j in range(K):
                q = 0
                for t in range(b):
                    p = j * b + t
                    q |= ((row[p // 8] >> (p % 8)) & 1) << t
                if enc["fmt"] == "uniform":
                    g = j // enc["group"]
                    d = float(enc["scales"][i, g]) * (q - float(enc["zeros"][i, g]))
                elif enc["fmt"] == "bpdq":
                    c = [float(v) for v in enc["coefs"][i, j // enc["group"]]]
                    d = c[0]
                    for t in range(b):  # plane t+1 is bit t of the code
                        if (q >> t) & 1:
                            d += c[t + 1]
                else:
                    d = float(enc["lut"][i, q])
                acc += d * x[j]
            for p in range(int(rp[i]), int(rp[i + 1])):
                acc += float(va[p]) * x[int(ci[p])]
            y.append(acc)
        Y.append(y)
    return np.array(Y)


def _tiny_enc(bits, fmt, n_out, seed, M=6, K=64, B=2):
    rng = np.random.default_rng(seed)
    W = (0.02 * rng.standard_normal((M, K))).astype(np.float16)
    idx = rng.choice(M * K, size=n_out, replace=False)
    W.ravel()[idx] = rng.uniform(0.3, 2.0, size=n_out) * np.where(rng.integers(0, 2, n_out) > 0, 1, -1)
    x = rng.standard_normal((B, K)).astype(np.float16)
    group = 32 if fmt == "bpdq" else 16
    enc = encode.encode(W, bits, fmt, n_out, group, sens=x[0].astype(np.float64) ** 2)
    return W, x, enc


def check_brute_force(enc, x):
    y, A = gemv.gemv(enc, x)
    yb = brute_force_y(enc, x)
    return bool(np.all(np.abs(y - yb) <= 1e-12 * (A + 1.0)))


@pytest.mark.parametrize("bits,fmt", [(3, "uniform"), (4, "uniform"), (3, "lut"), (4, "lut"), (3, "bpdq")])
@pytest.mark.parametrize("n_out", [0, 5])
def test_gemv_matches_brute_force(bits, fmt, n_out):
    W, x, enc = _tiny_enc(bits, fmt, n_out, seed=bits * 10 + n_out)
    assert check_brute_force(enc, x)


def test_brute_force_catches_dropped_sparse_term(monkeypatch):
    W, x, enc = _tiny_enc(3, "uniform", 5, seed=7)
    monkeypatch.setattr(gemv, "sparse_rows",
                        lambda e, rows: (np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0)))
    assert not check_brute_force(enc, x)


def test_brute_force_catches_zero_sign(monkeypatch):
    W, x, enc = _tiny_enc(4, "uniform", 5, seed=8)
    orig = gemv.decode_rows

    def plus_z(e, rows=None, codes=None):
        e2 = dict(e)
        e2["zeros"] = (-e["zeros"].astype(np.float64)).astype(np.float16)
        return orig(e2, rows, codes)
    monkeypatch.setattr(gemv, "decode_rows", plus_z)
    assert not check_brute_force(enc, x)


def test_brute_force_catches_transposed_lut(monkeypatch):
    W, x, enc = _tiny_enc(3, "lut", 5, seed=9)
    orig = gemv.decode_rows

    def reversed_lut(e, rows=None, codes=None):
        e2 = dict(e)
        e2["lut"] = e["lut"][:, ::-1].copy()
        return orig(e2, rows, codes)
    monkeypatch.setattr(gemv, "decode_rows", reversed_lut)
    assert not check_brute_force(enc, x)


def test_brute_force_catches_reversed_bit_planes(monkeypatch):
    W, x, enc = _tiny_enc(3, "bpdq", 5, seed=10)
    orig = gemv.decode_rows

    def reversed_planes(e, rows=None, codes=None):
        e2 = dict(e)
        c = e["coefs"].copy()
        c[:, :, 1:] = c[:, :, :0:-1]
        e2["coefs"] = c
        return orig(e2, rows, codes)
    monkeypatch.setattr(gemv, "decode_rows", reversed_planes)
    assert not check_brute_force(enc, x)


def test_zero_outlier_case_is_plain_dequant_gemv():
    """With no outliers the CSR is empty and y = D x exactly as a dense product."""
    for bits, fmt in [(3, "uniform"), (4, "lut")]:
        W, x, enc = _tiny_enc(bits, fmt, 0, seed=11)
        assert enc["row_ptr"].tolist() == [0] * (enc["M"] + 1)
        assert len(enc["col_idx"]) == 0 and len(enc["values"]) == 0
        D = gemv.decode(enc)
        y, _ = gemv.gemv(enc, x)
        assert np.array_equal(y, x.astype(np.float64) @ D.T)


def test_sparse_scatter_equals_dense_product():
    """y = (D + scatter(CSR)) x, using a dense fp64 product of the summed matrix."""
    for name in ["tiny_u4", "mlp7b_lut3"]:
        wl, W, planted, x, enc = small(name)
        D = gemv.decode(enc)
        S = gemv.sparse_dense(enc)
        y, A = gemv.gemv(enc, x)
        y2 = x.astype(np.float64) @ (D + S).T
        assert np.all(np.abs(y - y2) <= 1e-12 * (A + 1.0))
        # and dense + sparse equals W wherever it is an outlier, decoded dense elsewhere
        assert np.array_equal((D + S)[planted], W.astype(np.float64)[planted])


# ---------------------------------------------------------------------------
# Pin 3b: the acceptance test -- the tolerance scale A and the bound
# ---------------------------------------------------------------------------
def loop_weights(enc):
    """Effective weights w_ij = d_ij + (CSR entry at (i, j)) in pure Python,
    each code read bit by bit from the canonical bytes (no numpy arithmetic)."""
    M, K, b = enc["M"], enc["K"], enc["bits"]
    packed = np.asarray(enc["codes_packed"])
    rp, ci, va = enc["row_ptr"], enc["col_idx"], enc["values"]
    W = []
    for i in range(M):
        row = [int(v) for v in packed[i]]
        w = []
        for j in range(K):
            q = 0
            for t in range(b):
                p = j * b + t
                q |= ((row[p // 8] >> (p % 8)) & 1) << t
            if enc["fmt"] == "uniform":
                g = j // enc["group"]
                d = float(enc["scales"][i, g]) * (q - float(enc["zeros"][i, g]))
            elif enc["fmt"] == "bpdq":
                c = [float(v) for v in enc["coefs"][i, j // enc["group"]]]
                d = c[0] + sum(c[t + 1] for t in range(b) if (q >> t) & 1)
            else:
                d = float(enc["lut"][i, q])
            w.append(d)
        for p in range(int(rp[i]), int(rp[i + 1])):
            w[int(ci[p])] += float(va[p])
        W.append(w)
    return W


def loop_tolerance_scale(W, X16):
    """A[b][i] = sum_j |w_ij * x_bj|, one term at a time."""
    return np.array([[sum(abs(wij * float(xj)) for wij, xj in zip(wi, xb)) for wi in W] for xb in np.asarray(X16)])


def check_tolerance_scale(enc, x):
    _, A = gemv.gemv(enc, x)
    Al = loop_tolerance_scale(loop_weights(enc), x)
    return bool(np.all(np.abs(A - Al) <= 1e-12 * Al + 1e-300))


@pytest.mark.parametrize("bits,fmt", [(3, "uniform"), (4, "uniform"), (3, "lut"), (4, "lut"), (3, "bpdq")])
@pytest.mark.parametrize("n_out", [0, 5])
def test_tolerance_scale_matches_loop(bits, fmt, n_out):
    """A = sum_j |w_ij x_j| over the weights the product uses (dense decode plus CSR)."""
    W, x, enc = _tiny_enc(bits, fmt, n_out, seed=bits * 10 + n_out + 100)
    assert check_tolerance_scale(enc, x)
    # also on a row subset, the way the GPU tests call it
    rows = np.array([1, 4])
    _, A = gemv.gemv_rows(enc, x, rows)
    Al = loop_tolerance_scale(loop_weights(enc), x)[:, rows]
    assert np.all(np.abs(A - Al) <= 1e-12 * Al)


def test_tolerance_scale_catches_abs_of_product(monkeypatch):
    """|sum_j w_ij x_j| in place of sum_j |w_ij x_j|."""
    W, x, enc = _tiny_enc(4, "lut", 5, seed=31)

    def abs_of_product(xx, D, loc, col, val):
        Wd = np.array(D, copy=True)
        np.add.at(Wd, (loc, col), val)
        return np.abs(xx @ Wd.T)
    monkeypatch.setattr(gemv, "tolerance_scale", abs_of_product)
    assert not check_tolerance_scale(enc, x)


def test_tolerance_scale_catches_dropped_sparse_term(monkeypatch):
    W, x, enc = _tiny_enc(3, "uniform", 5, seed=32)
    monkeypatch.setattr(gemv, "tolerance_scale", lambda xx, D, loc, col, val: np.abs(xx) @ np.abs(D).T)
    assert not check_tolerance_scale(enc, x)


def test_tolerance_scale_at_a_shared_position():
    """A dense value 0.5 everywhere and a CSR entry -0.25 at column 3 (w = 0.25 there):
    with x = 1, A = 31 * 0.5 + 0.25 = 15.75 (summing |d x| and |r x| apart would give 16.25)."""
    K = 32
    codes = np.full((1, K), 5, dtype=np.uint8)
    lut = np.zeros((1, 16), np.float16)
    lut[0, 5] = 0.5
    enc = {"M": 1, "K": K, "bits": 4, "fmt": "lut", "group": 0, "codes": codes,
           "codes_packed": pack.pack_bitstream(codes, 4), "lut": lut,
           "row_ptr": np.array([0, 1], np.int32), "col_idx": np.array([3], np.int32),
           "values": np.array([-0.25], np.float16)}
    y, A = gemv.gemv(enc, np.ones((1, K), np.float16))
    assert y[0, 0] == 15.75 and A[0, 0] == 15.75
    x = np.ones((1, K), np.float16)
    x[0, 3] = -1
    y, A = gemv.gemv(enc, x)
    assert y[0, 0] == 15.25 and A[0, 0] == 15.75


def check_acceptance(within):
    """The bound |y_test - y| <= 1e-4 A + 1e-6, at hand-computed points on both sides of it."""
    A = np.array([0.0, 1.0, 2.0e4, 3.5])
    y = np.array([0.25, -1.0, 7.0, 0.0])
    bound = np.array([1e-6, 1.01e-4, 2.000001, 3.51e-4])
    inside = y + bound * (1 - 1e-6)
    outside = y - bound * (1 + 1e-6)
    ok_in, worst_in = within(inside, y, A)
    ok_out, worst_out = within(outside, y, A)
    one_out = inside.copy()
    one_out[1] = y[1] + 1.02e-4
    ok_one, worst_one = within(one_out, y, A)
    return (ok_in and worst_in <= 1.0 and not ok_out and worst_out > 1.0
            and not ok_one and abs(worst_one - 1.02e-4 / 1.01e-4) < 1e-9)


def test_acceptance_bound():
    assert check_acceptance(gemv.within_tolerance)


def test_acceptance_bound_catches_loose_rel():
    assert not check_acceptance(lambda yt, yr, A: gemv.within_tolerance(yt, yr, A, rel=1e-3))


def test_acceptance_bound_catches_missing_abs_term():
    assert not check_acceptance(lambda yt, yr, A: gemv.within_tolerance(yt, yr, A, abs_=0.0))


# ---------------------------------------------------------------------------
# Pin 4: canonical bitstream
# ---------------------------------------------------------------------------
def check_bitstream_golden():
    g = _golden("bitstream_lsb_first.json")
    for case in g["cases"]:
        codes = np.array([case["codes"]], dtype=np.uint8)
        got = pack.pack_bitstream(codes, case["bits"])[0]
        if [int(v) for v in got] != [int(c, 16) for c in case["bytes"]]:
            return False
        if not np.array_equal(pack.unpack_bitstream(got[None, :], case["bits"], codes.shape[1]), codes):
            return False
    return True


def test_bitstream_golden():
    assert check_bitstream_golden()


def test_bitstream_golden_catches_msb_first(monkeypatch):
    def msb_first(codes, bits):
        M, K = codes.shape
        planes = (codes[:, :, None].astype(np.uint16) >> np.arange(bits)[::-1]) & 1
        return np.packbits(planes.reshape(M, K * bits).astype(np.uint8), axis=1, bitorder="big")
    monkeypatch.setattr(pack, "pack_bitstream", msb_first)
    assert not check_bitstream_golden()


@pytest.mark.parametrize("bits", [3, 4])
def test_bitstream_roundtrip_every_value_every_offset(bits):
    K = 32 * (1 << bits)
    # every code value appears at every position of a 32-code (whole-dword) period
    codes = np.array([[(j + r) % (1 << bits) for j in range(K)] for r in range(1 << bits)], dtype=np.uint8)
    packed = pack.pack_bitstream(codes, bits)
    assert packed.shape == (1 << bits, K * bits // 8)
    assert np.array_equal(pack.unpack_bitstream(packed, bits, K), codes)


def test_bitstream_row_stride():
    codes = np.random.default_rng(3).integers(0, 8, size=(5, 64)).astype(np.uint8)
    packed = pack.pack_bitstream(codes, 3)
    for i in range(5):
        assert np.array_equal(packed[i], pack.pack_bitstream(codes[i:i + 1], 3)[0])


# ---------------------------------------------------------------------------
# Pin 5: uniform group quantization
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_u4", "attn7b_u3", "block7b_u3"])
def test_uniform_codes_are_nearest_grid_points(name):
    wl, W, planted, x, enc = small(name)
    L = (1 << wl.bits) - 1
    w = W.astype(np.float64)
    s = np.repeat(enc["scales"].astype(np.float64), wl.group, axis=1)
    z = np.repeat(enc["zeros"].astype(np.float64), wl.group, axis=1)
    grid = s[..., None] * (np.arange(L + 1)[None, None, :] - z[..., None])   # [M, K, L+1]
    best = np.min(np.abs(w[..., None] - grid), axis=2)
    D = gemv.decode(enc)
    inl = ~planted
    # the chosen code is a nearest grid point (rint ties may pick either neighbour)
    assert np.all(np.abs(w - D)[inl] <= best[inl] + 1e-15)
    assert np.all(enc["codes"] <= L)
    # zero points are exact integers in [0, L]
    zz = enc["zeros"].astype(np.float64)
    assert np.array_equal(zz, np.rint(zz)) and zz.min() >= 0 and zz.max() <= L


@pytest.mark.parametrize("name", ["tiny_u4", "attn7b_u3"])
def test_uniform_error_bound(name):
    """|w - d| <= scale/2 + L*|scale - (hi - lo)/L| for every non-outlier."""
    wl, W, planted, x, enc = small(name)
    L = (1 << wl.bits) - 1
    g = wl.group
    w = W.astype(np.float64).reshape(W.shape[0], -1, g)
    h = planted.reshape(w.shape)
    lo = np.minimum(0, np.where(h, np.inf, w).min(axis=2))
    hi = np.maximum(0, np.where(h, -np.inf, w).max(axis=2))
    s = enc["scales"].astype(np.float64)
    bound = s / 2 + L * np.abs(s - (hi - lo) / L)
    err = np.abs(w - gemv.decode(enc).reshape(w.shape))
    assert np.all(np.where(h, 0, err) <= bound[..., None] + 1e-15)


def test_uniform_exact_on_grid():
    """Weights that already lie on a representable grid decode exactly."""
    rng = np.random.default_rng(5)
    scale = 2.0 ** -7
    q = rng.integers(0, 16, size=(4, 64))
    z = 5
    q[:, ::16] = 0      # make every group span the full code range
    q[:, 1::16] = 15
    W = (scale * (q - z)).astype(np.float16)
    enc = encode.encode(W, 4, "uniform", 0, 16)
    assert np.array_equal(gemv.decode(enc), W.astype(np.float64))
    assert np.all(enc["scales"].astype(np.float64) == scale)
    assert np.all(enc["zeros"].astype(np.float64) == z)


# ---------------------------------------------------------------------------
# Pin 6: weighted Lloyd-Max
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_lloyd_objective_never_increases(seed):
    rng = np.random.default_rng(seed)
    w = 0.02 * rng.standard_normal(500)
    s = rng.standard_normal(500) ** 2
    hist = []
    cent, zi = encode.lloyd_row(w, s, 8, history=hist)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))
    assert cent[zi] == 0.0 and np.all(np.diff(cent) >= 0)


@pytest.mark.parametrize("seed", range(4))
def test_lloyd_terminates_at_fixed_point(seed):
    rng = np.random.default_rng(100 + seed)
    w = 0.02 * rng.standard_normal(300)
    s = rng.uniform(0.1, 3.0, 300)
    cent, zi = encode.lloyd_row(w, s, 16)
    a = encode.nearest(w, cent)
    for c in range(16):
        if c == zi or not np.any(a == c):
            continue
        mean = np.sum(s[a == c] * w[a == c]) / np.sum(s[a == c])
        assert abs(mean - cent[c]) <= 1e-15 * max(1.0, abs(mean)) + 1e-18


def _brute_force_pinned_optimum(w, s, C):
    """Global optimum over every assignment of points to C clusters, one pinned at 0."""
    import itertools
    best = np.inf
    n = len(w)
    for assign in itertools.product(range(C), repeat=n):
        a = np.array(assign)
        sse = 0.0
        for c in range(C):
            sel = a == c
            if not sel.any():
                continue
            if c == 0:
                sse += np.sum(s[sel] * w[sel] ** 2)
            else:
                m = np.sum(s[sel] * w[sel]) / np.sum(s[sel])
                sse += np.sum(s[sel] * (w[sel] - m) ** 2)
        best = min(best, sse)
    return best


@pytest.mark.parametrize("seed", range(3))
def test_lloyd_not_below_global_optimum(seed):
    rng = np.random.default_rng(200 + seed)
    w = rng.standard_normal(7)
    s = rng.uniform(0.2, 2.0, 7)
    cent, zi = encode.lloyd_row(w, s, 3)
    a = encode.nearest(w, cent)
    sse = encode.weighted_sse(w, s, cent, a)
    opt = _brute_force_pinned_optimum(w, s, 3)
    assert sse >= opt - 1e-12


def test_lloyd_recovers_exact_clusters():
    """Data made of C-1 distinct values with equal mass are reproduced exactly."""
    vals = np.array([-0.75, -0.5, -0.25, 0.125, 0.25, 0.5, 1.0])
    w = np.repeat(vals, 8)
    s = np.ones_like(w)
    cent, zi = encode.lloyd_row(w, s, 8)
    assert sorted(set(cent.tolist()) - {0.0}) == sorted(vals.tolist())
    W = np.tile(w, (2, 1)).astype(np.float16)
    enc = encode.encode(W, 3, "lut", 0, sens=np.ones(W.shape[1]))
    assert np.array_equal(gemv.decode(enc), W.astype(np.float64))


def check_weighted_quantile(wq):
    """Lower inverse CDF of the weighted sample, at hand-computed levels.

    w = (3, 1, 2, 5) with weights (1, 1, 2, 0): sorted 1, 2, 3, 5 with
    cumulative fractions 0.25, 0.75, 1, 1.
    """
    w = np.array([3.0, 1.0, 2.0, 5.0])
    s = np.array([1.0, 1.0, 2.0, 0.0])
    got = wq(w, s, [0.1, 0.25, 0.26, 0.75, 0.9, 1.0])
    if got.tolist() != [1.0, 1.0, 2.0, 2.0, 3.0, 3.0]:
        return False
    # equal weights: the level 1/2 of 1..5 is the lower median
    return wq(np.arange(1.0, 6.0), np.ones(5), [0.5]).tolist() == [3.0]


def test_weighted_quantile_pin():
    assert check_weighted_quantile(encode.weighted_quantile)


def test_weighted_quantile_catches_upper_inverse():
    def upper(w, s, qs):
        order = np.argsort(w, kind="stable")
        cw = np.cumsum(s[order]) / s.sum()
        idx = np.searchsorted(cw, np.asarray(qs, dtype=np.float64), side="right")
        return w[order][np.minimum(idx, len(w) - 1)]
    assert not check_weighted_quantile(upper)


def test_weighted_quantile_catches_dropped_weights():
    assert not check_weighted_quantile(lambda w, s, qs: encode.weighted_quantile(w, np.ones_like(s), qs))


def check_lloyd_first_steps(lloyd):
    """Initialisation at the weighted levels (k + 1/2)/(C - 1) and one
    assign-and-update step, by hand, on w = 1..12.

    Equal weights, C = 4: the levels 1/6, 1/2, 5/6 give the free centroids
    2, 6, 10 next to the pinned 0.  One step: 1 ties between 0 and 2 and goes
    to 0 (the lower), 2, 3, 4 (tie) go to 2, 5..8 (8 ties) to 6, 9..12 to 10;
    the new centroids are the means 3, 6.5 and 10.5.  With weight 3 on w = 4
    the first free centroid moves to (2 + 3 + 12) / 5 = 3.4 instead, and with
    weight 11 on w = 12 (and 1 elsewhere) the initial free centroids are 4,
    11 and 12.
    """
    w = np.arange(1.0, 13.0)
    ones = np.ones(12)
    init, _ = lloyd(w, ones, 4, max_iter=0)
    one, _ = lloyd(w, ones, 4, max_iter=1)
    s4 = ones.copy()
    s4[3] = 3.0
    one4, _ = lloyd(w, s4, 4, max_iter=1)
    s12 = ones.copy()
    s12[11] = 11.0
    init12, _ = lloyd(w, s12, 4, max_iter=0)
    return (init.tolist() == [0.0, 2.0, 6.0, 10.0] and one.tolist() == [0.0, 3.0, 6.5, 10.5]
            and abs(one4[1] - 3.4) < 1e-12 and init12.tolist() == [0.0, 4.0, 11.0, 12.0])


def test_lloyd_first_steps_pin():
    assert check_lloyd_first_steps(encode.lloyd_row)


def test_lloyd_first_steps_catch_levels_without_the_half(monkeypatch):
    orig = encode.weighted_quantile
    monkeypatch.setattr(encode, "weighted_quantile",
                        lambda w, s, qs: orig(w, s, np.asarray(qs) - 0.5 / (len(qs))))
    assert not check_lloyd_first_steps(encode.lloyd_row)


def test_lloyd_first_steps_catch_unweighted_update():
    def unweighted(w, s, C, max_iter=100, history=None):
        # the oracle's own steps with the mean update dropping the weights
        cent, zi = encode.lloyd_row(w, s, C, max_iter=0)
        for _ in range(max_iter):
            a = encode.nearest(w, cent)
            for c in range(C):
                if c != zi and np.any(a == c):
                    cent[c] = w[a == c].mean()
        return cent, zi
    assert not check_lloyd_first_steps(unweighted)


def test_lut_codes_nearest_and_zero_pinned():
    wl, W, planted, x, enc = small("mlp7b_lut3")
    lut = enc["lut"].astype(np.float64)
    assert np.all(np.diff(lut, axis=1) >= 0)
    assert np.all(np.any(lut == 0.0, axis=1))
    w = W.astype(np.float64)
    dist = np.abs(w[:, :, None] - lut[:, None, :])
    D = gemv.decode(enc)
    inl = ~planted
    assert np.all(np.abs(w - D)[inl] == dist.min(axis=2)[inl])
    assert np.all(D[planted] == 0.0)


# ---------------------------------------------------------------------------
# Pin 7: bit accounting against the pages' orders of magnitude
# ---------------------------------------------------------------------------
def test_extra_bits_per_weight_one_percent():
    """[SpQR] about 1 % FP16 outliers + index overhead = roughly 0.5-1 extra bit per weight."""
    for name, layer in [("tiny_u4", 0), ("block7b_u3", 0), ("block7b_u3", 6)]:
        wl = WORKLOADS[name]
        M, K = (wl.layers[layer][1:] if wl.layers else (wl.M, wl.K))
        nnz = outlier_count(wl, M, K)
        bpw = accounting.sparse_bpw(M, K, nnz)
        assert 0.45 <= bpw <= 1.0, (name, bpw)
    assert abs(accounting.sparse_bpw(512, 512, 2621) - 0.5425) < 1e-4


def test_extra_bits_per_weight_squeezellm_order_of_magnitude():
    """[SqLLM] ~0.45 % outliers cost about 0.1 bit/weight: same order of magnitude."""
    wl = WORKLOADS["mlp7b_lut3"]
    nnz = outlier_count(wl, wl.M, wl.K)
    assert nnz == 202899
    for col_bytes in (2, 4):
        bpw = accounting.sparse_bpw(wl.M, wl.K, nnz, col_bytes=col_bytes)
        assert 0.05 < bpw < 0.5
    assert accounting.dense_bpw(3, "lut", 4096) == pytest.approx(3.03125)
    assert accounting.dense_bpw(3, "uniform", 4096, 16) == 5.0


# ---------------------------------------------------------------------------
# Sensitivity-based outlier pick ([SqLLM] "Sélection des outliers")
# ---------------------------------------------------------------------------
def _loop_first_pass_error(W16, sens, bits):
    """s_j (w - q(w))^2 with q the nearest entry of the row's FP16 first-pass table, by plain loops."""
    M, K = W16.shape
    W = W16.astype(np.float64)
    out = np.zeros((M, K))
    for i in range(M):
        cent, _ = encode.lloyd_row(W[i], np.asarray(sens, np.float64), 1 << bits)
        tab = sorted(float(v) for v in cent.astype(np.float16))
        for j in range(K):
            best = min(tab, key=lambda c: abs(W[i, j] - c))
            out[i, j] = sens[j] * (W[i, j] - best) ** 2
    return out


def check_pick_minimizes_remaining_error(W16, sens, bits, n):
    """Extracting the picked weights leaves the least weighted first-pass error of
    all n-subsets: the pages' picked weights carry most of the potential error."""
    import itertools
    e = _loop_first_pass_error(W16, sens, bits).ravel()
    mask = encode.pick_outliers_sensitivity(W16, sens, bits, n).ravel()
    assert mask.sum() == n
    got = e[~mask].sum()
    best = min(e.sum() - sum(e[list(c)]) for c in itertools.combinations(range(e.size), n))
    assert got <= best + 1e-15 * max(1.0, abs(best)), (got, best)


@pytest.mark.parametrize("seed", range(3))
def test_sensitivity_pick_minimizes_remaining_error(seed):
    rng = np.random.default_rng(seed)
    W16 = (rng.standard_normal((2, 8)) * 0.05).astype(np.float16)
    sens = rng.uniform(0.0, 3.0, size=8)
    check_pick_minimizes_remaining_error(W16, sens, 2, 3)


def test_sensitivity_pick_catches_smallest_first(monkeypatch):
    orig = encode.first_pass_error
    monkeypatch.setattr(encode, "first_pass_error", lambda W, s, b: -orig(W, s, b))
    rng = np.random.default_rng(0)
    W16 = (rng.standard_normal((2, 8)) * 0.05).astype(np.float16)
    with pytest.raises(AssertionError):
        check_pick_minimizes_remaining_error(W16, rng.uniform(0.0, 3.0, size=8), 2, 3)


def _moderate_vs_large_row():
    """One row: a bulk of N(0, 0.02) weights of sensitivity 1, twelve large
    weights (0.5 .. 2.5) in columns of sensitivity 1e-6, and ten moderate
    weights (-0.1 .. 0.1) in columns of sensitivity 100.  Each group outnumbers
    the seven free entries of a 3-bit table, so neither can be fitted exactly."""
    rng = np.random.default_rng(5)
    K = 128
    w = rng.standard_normal(K) * 0.02
    s = np.ones(K)
    lo = np.arange(40, 52)
    w[lo] = np.linspace(0.5, 2.5, lo.size)
    s[lo] = 1e-6
    hi = np.arange(20, 30)
    w[hi] = np.linspace(-0.1, 0.1, hi.size)
    s[hi] = 100.0
    return w.astype(np.float16)[None, :], s, hi, lo


def check_moderate_high_sensitivity_picked(pick):
    W16, s, hi, lo = _moderate_vs_large_row()
    m = pick(W16, s, 3, 2)[0]
    assert not m[lo].any(), "a large weight of negligible sensitivity was taken"
    assert set(np.flatnonzero(m)) <= set(hi), "a pick is not a moderate weight of high sensitivity"


def test_sensitivity_pick_takes_moderate_weight_of_high_sensitivity():
    check_moderate_high_sensitivity_picked(encode.pick_outliers_sensitivity)
    # the magnitude pick takes large weights instead
    W16, s, hi, lo = _moderate_vs_large_row()
    assert set(np.flatnonzero(encode.pick_outliers(W16, 2)[0])) <= set(lo)


def test_sensitivity_pick_catches_dropped_sensitivity(monkeypatch):
    orig = encode.first_pass_error
    monkeypatch.setattr(encode, "first_pass_error", lambda W, s, b: orig(W, np.ones_like(s), b))
    with pytest.raises(AssertionError):
        check_moderate_high_sensitivity_picked(encode.pick_outliers_sensitivity)


def test_sensitivity_pick_equal_sensitivity_takes_planted():
    """With equal sensitivities the criterion is the plain squared error: with
    twenty planted weights in 0.5 .. 2.5 per row, more than a 3-bit table can
    fit, the twelve picked per row are all planted ones."""
    rng = np.random.default_rng(2)
    M, K = 3, 512
    W = rng.standard_normal((M, K)) * 0.02
    planted = np.zeros((M, K), dtype=bool)
    for i in range(M):
        cols = rng.choice(K, size=20, replace=False)
        W[i, cols] = rng.uniform(0.5, 2.5, size=20) * rng.choice([-1.0, 1.0], size=20)
        planted[i, cols] = True
    m = encode.pick_outliers_sensitivity(W.astype(np.float16), np.ones(K), 3, 12 * M)
    assert m.sum() == 12 * M
    assert not (m & ~planted).any()


def test_sensitivity_pick_encoding_is_exact_at_outliers():
    """The encoding built on the sensitivity pick keeps the pages' invariants:
    holes decode to 0 and dense + sparse reproduces every outlier exactly."""
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, 24, 256)
    x = make_x(wl, 1, 256, 0, 24)
    n = 40
    enc = encode.encode(W, 3, "lut", n, sens=x[0].astype(np.float64) ** 2, pick="sensitivity")
    assert int(enc["row_ptr"][-1]) == n
    check_exact_outliers(W, enc)


# ---------------------------------------------------------------------------
# SSQR: overflow-tolerant uniform grids ([Babai/GPTQ] "3. Applications
# Pratiques et Algorithmes")
# ---------------------------------------------------------------------------
def _ssqr_matrix(seed=0, M=8, K=64):
    wl = WORKLOADS["attn7b_u3"]
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((M, K)) * 0.02
    idx = rng.choice(M * K, size=6, replace=False)
    W.flat[idx] = rng.uniform(0.3, 1.5, size=6) * rng.choice([-1.0, 1.0], size=6)
    return W.astype(np.float16)


def check_ssqr_grid(W16, bits, alpha):
    """Inliers sit on the nearest point of their group's grid; overflows are
    exactly the weights whose nearest grid point lies outside [0, 2^b - 1]."""
    codes, scales, zeros, over = encode.quant_uniform_scaled(W16, bits, 16, alpha)
    L = (1 << bits) - 1
    M, K = W16.shape
    w = W16.astype(np.float64)
    for i in range(M):
        for j in range(K):
            s = float(scales[i, j // 16]); z = float(zeros[i, j // 16])
            u = w[i, j] / s + z  # position on the integer grid
            if over[i, j]:
                assert u < -0.5 or u > L + 0.5, (i, j, u)
                assert codes[i, j] == z
            else:
                assert 0 <= codes[i, j] <= L
                assert abs(w[i, j] - s * (codes[i, j] - z)) <= 0.5 * s + 1e-12 * abs(w[i, j]), (i, j)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("alpha", [1.0, 0.6, 0.25])
def test_ssqr_inliers_on_grid_overflows_outside(bits, alpha):
    check_ssqr_grid(_ssqr_matrix(bits), bits, alpha)


def test_ssqr_grid_catches_floor(monkeypatch):
    monkeypatch.setattr(encode.np, "rint", np.floor)
    with pytest.raises(AssertionError):
        check_ssqr_grid(_ssqr_matrix(1), 3, 0.6)


def check_ssqr_budget(W16, bits, n):
    """The search keeps the overflow count within the budget, with the finest
    grids that do: one search step lower, the budget is exceeded."""
    a = encode.ssqr_alpha(W16, bits, 16, n)
    count = lambda t: int(encode.quant_uniform_scaled(W16, bits, 16, t)[3].sum())
    assert count(a) <= n
    assert count(a - 2.0 ** -38) > n


@pytest.mark.parametrize("n", [0, 3, 6, 40])
def test_ssqr_search_meets_budget(n):
    check_ssqr_budget(_ssqr_matrix(2), 3, n)


def test_ssqr_search_catches_flipped_direction(monkeypatch):
    orig = encode.quant_uniform_scaled
    # a search that keeps the coarsest grid: report every overflow count as within budget
    monkeypatch.setattr(encode, "quant_uniform_scaled",
                        lambda W, b, g, a: orig(W, b, g, a)[:3] + (np.zeros(W.shape, dtype=bool),))
    W16 = _ssqr_matrix(2)
    with pytest.raises(AssertionError):
        a = encode.ssqr_alpha(W16, 3, 16, 3)
        assert orig(W16, 3, 16, a)[3].sum() <= 3


def test_ssqr_all_sparse_is_plain_product():
    """A budget of every weight: the grids shrink until all nonzero weights
    overflow, the dense part decodes to 0 and y is the plain FP16 product."""
    W16 = _ssqr_matrix(3)
    M, K = W16.shape
    enc = encode.encode(W16, 3, "uniform", M * K, pick="ssqr")
    assert np.all(gemv.decode(enc) == 0.0)
    x = np.random.default_rng(4).standard_normal((1, K)).astype(np.float16)
    y, _ = gemv.gemv_rows(enc, x)
    assert np.allclose(y, W16.astype(np.float64) @ x[0].astype(np.float64), rtol=0, atol=1e-12)


def test_ssqr_no_budget_all_inliers():
    W16 = _ssqr_matrix(4)
    enc = encode.encode(W16, 4, "uniform", 0, pick="ssqr")
    assert int(enc["row_ptr"][-1]) == 0
    check_ssqr_grid(W16, 4, enc["alpha"])


def test_ssqr_encoding_is_exact_at_outliers():
    W16 = _ssqr_matrix(5, M=16, K=128)
    enc = encode.encode(W16, 3, "uniform", 10, pick="ssqr")
    assert 0 < int(enc["row_ptr"][-1]) <= 10
    check_exact_outliers(W16, enc)



# ---------------------------------------------------------------------------
# BPDQ ([BPDQ] "1. Formulation de la Grille Variable", "2. Cadre d'Optimisation")
# ---------------------------------------------------------------------------
def test_bpdq_fit_one_plane_is_class_means():
    """With one plane the least-squares levels are the two class means:
    C0 = mean(w | b = 0), C1 = mean(w | b = 1) - C0."""
    rng = np.random.default_rng(0)
    w = rng.standard_normal(40)
    q = rng.integers(0, 2, size=40)
    c = encode.bpdq_fit(w, q, 1)
    m0, m1 = w[q == 0].mean(), w[q == 1].mean()
    assert np.allclose(c, [m0, m1 - m0], rtol=0, atol=1e-12)


def test_bpdq_fit_catches_missing_intercept(monkeypatch):
    def no_intercept(w, q, k):
        A = np.stack([((q >> (i - 1)) & 1).astype(np.float64) for i in range(1, k + 1)], axis=1)
        return np.concatenate([[0.0], np.linalg.lstsq(A, w, rcond=None)[0]])
    monkeypatch.setattr(encode, "bpdq_fit", no_intercept)
    with pytest.raises(AssertionError):
        test_bpdq_fit_one_plane_is_class_means()


def check_bpdq_assign_is_enumeration(assign):
    """Each weight takes the bit pattern whose level C0 + sum_i C_i b_i is nearest,
    found by listing all patterns (ties: lower code)."""
    rng = np.random.default_rng(1)
    k = 3
    c = rng.standard_normal(k + 1) * 0.05
    w = rng.standard_normal(200) * 0.1
    q = assign(w, c, k)
    for j in range(w.size):
        best, bq = None, None
        for code in range(1 << k):
            lv = c[0] + sum(c[i] for i in range(1, k + 1) if (code >> (i - 1)) & 1)
            e = abs(w[j] - lv)
            if best is None or e < best:
                best, bq = e, code
        assert q[j] == bq, (j, q[j], bq)


def test_bpdq_assign_is_enumeration():
    check_bpdq_assign_is_enumeration(encode.bpdq_assign)


def test_bpdq_assign_catches_msb_first_planes(monkeypatch):
    def msb_levels(c, k):
        q = np.arange(1 << k)
        return c[0] + sum(c[i] * ((q >> (k - i)) & 1) for i in range(1, k + 1))
    monkeypatch.setattr(encode, "bpdq_levels", msb_levels)
    with pytest.raises(AssertionError):
        check_bpdq_assign_is_enumeration(encode.bpdq_assign)


@pytest.mark.parametrize("seed", range(4))
def test_bpdq_objective_never_increases(seed):
    """Alternating exact bit updates and least-squares refits never raise the error."""
    rng = np.random.default_rng(seed)
    w = np.concatenate([rng.standard_normal(50) * 0.02, rng.standard_normal(14) * 0.08])
    hist = []
    encode.bpdq_group(w, 3, history=hist)
    assert len(hist) >= 1
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))


def test_bpdq_contains_uniform_grids():
    """The pages: the variable grid contains the uniform ones.  Weights on a
    uniform 3-bit grid (C_i = 2^(i-1) s) are reproduced exactly."""
    rng = np.random.default_rng(3)
    s, lo = 2.0 ** -7, -2.0 ** -4
    q = np.concatenate([np.arange(8), rng.integers(0, 8, size=56)])
    w = (lo + s * q).astype(np.float16).astype(np.float64)
    codes, c = encode.bpdq_group(w, 3)
    assert np.array_equal(encode.bpdq_levels(c, 3)[codes], w)


# ---------------------------------------------------------------------------
# HPTQ: Huffman-coded integers on one unconstrained grid
# ([Babai/GPTQ] "3. Applications Pratiques et Algorithmes")
# ---------------------------------------------------------------------------
from oracle import hptq  # noqa: E402


def _huffman_cost(freq):
    """Cost sum f_i l_i of an unlimited Huffman code, by repeatedly merging the two lightest."""
    import heapq
    h = [(float(f), i) for i, f in enumerate(freq)]
    heapq.heapify(h)
    cost, k = 0.0, len(freq)
    while len(h) > 1:
        a, _ = heapq.heappop(h)
        b, _ = heapq.heappop(h)
        cost += a + b
        heapq.heappush(h, (a + b, k)); k += 1
    return cost


def _best_limited_cost(freq, L):
    """Least sum f_i l_i over all length vectors with 1 <= l_i <= L and Kraft sum <= 1."""
    import itertools
    best = None
    for ls in itertools.product(range(1, L + 1), repeat=len(freq)):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            c = sum(f * l for f, l in zip(freq, ls))
            best = c if best is None or c < best else best
    return best


def check_package_merge(freq, L):
    ln = hptq.package_merge_lengths(np.asarray(freq, dtype=np.float64), L)
    assert ln.max() <= L
    assert abs(sum(2.0 ** -int(l) for l in ln) - 1.0) < 1e-12, "not a complete prefix code"
    assert sum(f * int(l) for f, l in zip(freq, ln)) == pytest.approx(_best_limited_cost(freq, L), abs=1e-9)


@pytest.mark.parametrize("freq,L", [([5, 1, 1, 2, 9], 4), ([1, 1, 2, 3, 5, 8], 3), ([1, 1, 2, 3, 5, 8], 5),
                                    ([4, 4, 4, 4], 2), ([7, 1], 1), ([3, 1, 1, 1, 1, 1], 3)])
def test_package_merge_is_optimal_within_limit(freq, L):
    check_package_merge(freq, L)


def test_package_merge_catches_keeping_one_item_too_many(monkeypatch):
    orig = hptq.package_merge_lengths

    def plus_one(freq, max_len):
        ln = orig(freq, max_len).copy()
        ln[int(np.argmin(ln))] += 1
        return ln
    monkeypatch.setattr(hptq, "package_merge_lengths", plus_one)
    with pytest.raises(AssertionError):
        check_package_merge([5, 1, 1, 2, 9], 4)


def test_package_merge_limit_binds_on_fibonacci_weights():
    freq = [1, 1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144]  # an unlimited Huffman code reaches length 11
    ln = hptq.package_merge_lengths(np.asarray(freq, float), 6)
    assert ln.max() <= 6
    assert abs(sum(2.0 ** -int(l) for l in ln) - 1.0) < 1e-12
    cost = sum(f * int(l) for f, l in zip(freq, ln))
    assert cost >= _huffman_cost(freq) - 1e-9
    assert hptq.package_merge_lengths(np.asarray(freq, float), 16).max() == 11
    assert sum(f * int(l) for f, l in zip(freq, hptq.package_merge_lengths(np.asarray(freq, float), 16))) \
        == pytest.approx(_huffman_cost(freq))


def check_canonical_prefix_free(sym, ln, codes):
    words = [format(int(c), f"0{int(l)}b") for c, l in zip(codes, ln)]
    for a in range(len(words)):
        for b in range(len(words)):
            if a != b:
                assert not words[b].startswith(words[a]), (words[a], words[b])


def test_canonical_code_is_prefix_free_and_round_trips():
    rng = np.random.default_rng(0)
    q = np.rint(rng.standard_normal((6, 256)) * 3).astype(np.int64)
    q[2, 7] = 40  # a rare large integer
    sym, ln, codes = hptq.build_code(q)
    check_canonical_prefix_free(sym, ln, codes)
    stream, row_bits = hptq.encode_stream(q, sym, ln, codes)
    assert row_bits[-1] == sum(int(ln[list(sym).index(v)]) for v in q.ravel())
    assert np.array_equal(hptq.decode_stream(stream, row_bits, 256, sym, ln, codes), q)


def test_canonical_code_catches_wrong_increment(monkeypatch):
    def bad(symbols, lengths):
        order = np.lexsort((symbols, lengths))
        s_, l_ = symbols[order], lengths[order]
        c = np.zeros(len(s_), dtype=np.int64)
        code, prev = 0, int(l_[0])
        for k in range(1, len(s_)):
            code = (code << (int(l_[k]) - prev)) + 1  # shift before the increment
            prev = int(l_[k])
            c[k] = code
        return s_, l_, c
    monkeypatch.setattr(hptq, "canonical_code", bad)
    q = np.array([[0, 0, 0, 1, 1, 2, 3, -1, -1, -1, -1, 4]], dtype=np.int64)
    with pytest.raises(AssertionError):
        check_canonical_prefix_free(*hptq.build_code(q))


def test_hptq_grid_has_no_clipping():
    """Every weight, outliers included, sits within half a step of its grid point."""
    wl = WORKLOADS["mlp7b_lut3"]
    W, planted = make_weights(wl, 0, 16, 512)
    s, q = hptq.grid(W, 128, 0.8)
    d = np.repeat(s, 128, axis=1) * q
    w = W.astype(np.float64)
    assert np.all(np.abs(w - d) <= 0.5 * np.repeat(s, 128, axis=1) * (1 + 1e-12))
    assert np.abs(q[planted]).min() > np.abs(q[~planted]).max() // 4  # outliers take large integers


def test_hptq_budget_boundary():
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, 8, 256)
    a = hptq.budget_alpha(W, 128, 3.125)
    bits = lambda t: hptq.stream_bits(hptq.grid(W, 128, t)[1])
    assert bits(a) <= 3.125 * W.size
    assert bits(a - 8.0 * 2.0 ** -40 * 4) > 3.125 * W.size


def test_hptq_gemv_matches_plain_product_of_decoded_grid():
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, 8, 256)
    enc = hptq.encode(W, 128, 3.125)
    x = np.random.default_rng(1).standard_normal((2, 256)).astype(np.float16)
    y, A = hptq.gemv(enc, x)
    d = np.repeat(enc["scales"].astype(np.float64), 128, axis=1) * enc["q"]
    assert np.allclose(y, x.astype(np.float64) @ d.T, rtol=0, atol=1e-12)


def string_prefix_decode(enc):
    """Integers read from the stream by matching codeword strings (the
    canonical codewords written out as '0'/'1' strings from the lengths)."""
    sym, ln, codes = hptq.canonical_code(np.asarray(enc["huff_sym"], np.int64), np.asarray(enc["huff_len"], np.int64))
    words = {format(int(c), f"0{int(l)}b"): int(s) for s, c, l in zip(sym, codes, ln)}
    bits = "".join(format(int(b), "08b") for b in np.asarray(enc["stream"], np.uint8))
    q = []
    for i in range(enc["M"]):
        p, row = int(enc["row_bits"][i]), []
        while len(row) < enc["K"]:
            w = ""
            while w not in words:
                w += bits[p]; p += 1
            row.append(words[w])
        assert p == int(enc["row_bits"][i + 1])
        q.append(row)
    return q


def check_hptq_gemv(enc, x):
    q = string_prefix_decode(enc)
    s = np.asarray(enc["scales"]).astype(np.float64)
    g = enc["group"]
    Wl = [[float(s[i, j // g]) * q[i][j] for j in range(enc["K"])] for i in range(enc["M"])]
    yl = np.array([[sum(w * float(v) for w, v in zip(wi, xb)) for wi in Wl] for xb in x])
    Al = loop_tolerance_scale(Wl, x)
    y, A = hptq.gemv(enc, x)
    rows = np.array([enc["M"] - 1, 0, 3])
    yr, Ar = hptq.gemv(enc, x, rows)
    return bool(np.all(np.abs(y - yl) <= 1e-12 * Al) and np.all(np.abs(A - Al) <= 1e-12 * Al)
                and np.all(np.abs(yr - yl[:, rows]) <= 1e-12 * Al[:, rows])
                and np.all(np.abs(Ar - Al[:, rows]) <= 1e-12 * Al[:, rows]))


def _hptq_tiny():
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, 6, 256)
    enc = hptq.encode(W, 128, 3.125)
    x = np.random.default_rng(4).standard_normal((2, 256)).astype(np.float16)
    return enc, x


def test_hptq_gemv_matches_string_decoder():
    """y and A of the HPTQ oracle against a decoder that matches codeword strings."""
    enc, x = _hptq_tiny()
    assert check_hptq_gemv(enc, x)


def test_hptq_gemv_catches_abs_of_product(monkeypatch):
    enc, x = _hptq_tiny()
    monkeypatch.setattr(gemv, "tolerance_scale", lambda xx, D, loc, col, val: np.abs(xx @ D.T))
    assert not check_hptq_gemv(enc, x)


def test_hptq_decode_rows_equals_whole_decode():
    """Rows decoded one at a time from their row_bits equal the same rows of the whole decode."""
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, 24, 256)
    enc = hptq.encode(W, 128, 3.125)
    full = hptq.decode(enc)
    rng = np.random.default_rng(2)
    for n in (1, 5, 24):
        rows = rng.choice(24, size=n, replace=False)
        assert np.array_equal(hptq.decode_rows(enc, rows), full[rows])
        assert np.array_equal(gemv.decode_rows(dict(enc, fmt="hptq"), rows), full[rows])
