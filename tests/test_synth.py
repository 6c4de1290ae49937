"""Seeded input generators: determinism, counts and the outlier structure of each workload."""

import numpy as np
import pytest

from synth import WORKLOADS, layer_shape, make_format_inputs, make_weights, make_x, outlier_count


def test_full_size_outlier_counts():
    expect = {"tiny_u4": 2621, "attn7b_u3": 83886, "mlp7b_lut3": 202899, "mlp70b_lut4": 1174405}
    for name, n in expect.items():
        wl = WORKLOADS[name]
        assert outlier_count(wl, wl.M, wl.K) == n
    wl = WORKLOADS["block7b_u3"]
    assert [outlier_count(wl, *layer_shape(wl, l)) for l in range(7)] == [167772] * 4 + [450888] * 3


def test_determinism_and_row0_of_x():
    a, pa = make_weights("attn7b_u3", 0, 32, 1024)
    b, pb = make_weights("attn7b_u3", 0, 32, 1024)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)) and np.array_equal(pa, pb)
    x1 = make_x("mlp70b_lut4", 1, 8192)
    x8 = make_x("mlp70b_lut4", 8, 8192)
    assert np.array_equal(x1[0].view(np.uint16), x8[0].view(np.uint16))
    assert x8.dtype == np.float16 and x8.shape == (8, 8192)


@pytest.mark.parametrize("name,M,K", [("tiny_u4", None, None), ("attn7b_u3", 64, 2048),
                                      ("mlp7b_lut3", 64, 1024), ("block7b_u3", 32, 1024)])
def test_planted_count_and_law(name, M, K):
    wl = WORKLOADS[name]
    W, planted = make_weights(wl, 0, M, K)
    M, K = W.shape
    assert planted.sum() == outlier_count(wl, M, K)
    a = np.abs(W.astype(np.float64))
    bulk = W.astype(np.float64)[~planted]
    assert bulk.std() == pytest.approx(wl.sigma, rel=0.05)
    if wl.law in ("top_bulk", "uniform_pos"):
        assert a[planted].min() >= 0.2 - 1e-3 and a[planted].max() <= 2.5 + 1e-3
    if wl.law == "student_t_top":
        assert a[planted].min() > 0.5


def test_row_skewed_structure():
    wl = WORKLOADS["mlp70b_lut4"]
    M, K = 400, 2048
    W, planted = make_weights(wl, 0, M, K)
    per_col = planted.sum(axis=0)
    full = np.flatnonzero(per_col == M)
    assert len(full) == 2
    per_row = planted.sum(axis=1) - 2
    heavy = per_row > 3 * np.median(per_row)
    assert heavy.sum() == int(np.floor(0.05 * M + 0.5))
    assert per_row[heavy].mean() / per_row[~heavy].mean() == pytest.approx(10.0, rel=0.1)
    assert planted.sum() == outlier_count(wl, M, K)


def test_format_inputs_shapes():
    f = make_format_inputs("mlp70b_lut4", 0, 64, 2048)
    assert f["codes_packed"].shape == (64, 1024) and f["lut"].shape == (64, 16)
    assert np.all(np.diff(f["lut"].astype(np.float64), axis=1) >= 0)
    assert np.all(np.any(f["lut"] == 0, axis=1))
    assert np.all(np.diff(f["rows"] * 2048 + f["cols"]) > 0)
    u = make_format_inputs("block7b_u3", 6)
    assert u["codes_packed"].shape == (4096, 11008 * 3 // 8) and u["scales"].shape == (4096, 688)
    z = u["zeros"].astype(np.float64)
    assert z.min() >= 0 and z.max() <= 7 and np.array_equal(z, np.rint(z))


def test_hptq_format_inputs_are_whole_rows_of_codewords():
    """The synthetic prefix code is a prefix code (Kraft sum <= 1), and the
    stream holds exactly the drawn integers, K per row (read back by the oracle)."""
    from oracle import hptq
    sym, ln, codes = __import__("synth").hptq_synthetic_code()
    assert sum(2.0 ** -int(l) for l in ln) <= 1.0
    f = make_format_inputs("mlp7b_hptq", 0, 40, 512)
    enc = dict(f, fmt="hptq")
    q = hptq.decode_stream(f["stream"], f["row_bits"], 512, *hptq.canonical_code(
        np.asarray(f["huff_sym"], np.int64), np.asarray(f["huff_len"], np.int64)))
    assert np.array_equal(q, f["q"])
    assert np.all(np.abs(f["q"]) <= 255)
    assert 2.8 < f["row_bits"][-1] / f["q"].size < 3.6
