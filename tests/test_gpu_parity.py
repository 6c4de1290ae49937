"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* Codes unpacked on the GPU from the repacked blob equal the oracle's codes
  bit-exactly.
* y satisfies |y_gpu - y| <= 1e-4 * sum_j |d_ij x_j| (+ sparse terms) + 1e-6 per output.
* Runs are bitwise deterministic and overwrite every output.

Small cases are oracle-encoded from the workloads' weight laws at sizes that
span several wave steps and a ragged tail.  Full sizes, every row, are in
test_gpu_parity_full.py.  Outputs are framed by canary words.
"""

import sys

import numpy as np
import pytest

from dense_sparse_bit_amd import qgemv
from gpu_checks import run_framed
from oracle import encode, gemv, pack
from synth import WORKLOADS, make_format_inputs, make_weights, make_x, outlier_count

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    return t


def csr_from_positions(M, rows, cols, values):
    counts = np.bincount(rows, minlength=M)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_ptr, cols.astype(np.int32), np.asarray(values, dtype=np.float16)


def format_case(name, layer=0, M=None, K=None):
    f = make_format_inputs(name, layer, M, K)
    f["row_ptr"], f["col_idx"], f["values"] = csr_from_positions(f["M"], f["rows"], f["cols"], f["values"])
    return f


_ENC = {}


def oracle_case(name, M, K, layer=0):
    key = (name, M, K, layer)
    if key not in _ENC:
        wl = WORKLOADS[name]
        W, planted = make_weights(wl, layer, M, K)
        M_, K_ = W.shape
        x = make_x(wl, max(wl.batches), K_, layer, M_)
        enc = encode.encode(W, wl.bits, wl.fmt, outlier_count(wl, M_, K_), wl.group or 16,
                            sens=x[0].astype(np.float64) ** 2)
        _ENC[key] = (enc, x)
    return _ENC[key]


def run_b1(torch, plan, x16):
    """Batch-1 run on the first row of x16, into a NaN-filled y framed by canaries."""
    return run_framed(torch, plan, x16[:1])


def run_bn(torch, plan, x16):
    """Batched run (B = rows of x16), into a NaN-filled y framed by canaries."""
    return run_framed(torch, plan, x16)


def check_y(y_gpu, enc, x16, rows=None):
    y_ref, A = gemv.gemv_rows(enc, x16[:y_gpu.shape[0]], rows)
    yg = y_gpu if rows is None else y_gpu[:, rows]
    assert np.all(np.isfinite(yg)), "output not fully written"
    ok, worst = gemv.within_tolerance(yg, y_ref, A)
    assert ok, f"tolerance exceeded: worst |dy|/(1e-4 A + 1e-6) = {worst:.3f}"
    return worst


SMALL_CASES = [
    ("tiny_u4", None, None),          # 512 x 512: one partial wave step (16 lanes)
    ("attn7b_u3", 200, 2080),         # one full step + a 1-lane tail
    ("attn7b_u3", 64, 4096),
    ("mlp7b_lut3", 64, 4096),
    ("mlp7b_lut3", 33, 4128),
    ("mlp70b_lut4", 24, 8192),        # 2 full outlier columns + heavy rows
    ("mlp70b_lut4", 40, 2080),
    ("block7b_u3", 96, 11008),        # down-proj K: 5 full steps + a 24-lane tail
    ("mlp7b_bpdq3", 64, 4096),        # BPDQ: 4 coefficients per row and group of 64
    ("mlp7b_bpdq3", 33, 2112),        # ragged M, a K-block half past K
]


@pytest.mark.parametrize("name,M,K", SMALL_CASES)
def test_small_oracle_encoded(torch, name, M, K):
    enc, x16 = oracle_case(name, M, K)
    _say(f"[gpu] small {name} M={enc['M']} K={enc['K']} nnz={enc['row_ptr'][-1]}")
    plan = qgemv.QGemv(enc)
    codes = plan.debug_unpack().cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(codes, enc["codes"]), "GPU-unpacked codes differ from the oracle's"
    y1 = run_b1(torch, plan, x16)
    check_y(y1, enc, x16)
    y2 = run_b1(torch, plan, x16)
    assert np.array_equal(y1, y2), "not bitwise deterministic"
    plan.close()


@pytest.mark.parametrize("name,M,K", [("mlp7b_lut3", 64, 4096), ("mlp70b_lut4", 40, 2080)])
def test_small_sensitivity_pick(torch, name, M, K):
    """Encodings whose outliers come from the sensitivity-weighted error pick."""
    wl = WORKLOADS[name]
    W, _ = make_weights(wl, 0, M, K)
    M_, K_ = W.shape
    x16 = make_x(wl, 1, K_, 0, M_)
    enc = encode.encode(W, wl.bits, wl.fmt, outlier_count(wl, M_, K_), 16,
                        sens=x16[0].astype(np.float64) ** 2, pick="sensitivity")
    _say(f"[gpu] sensitivity pick {name} M={M_} K={K_} nnz={enc['row_ptr'][-1]}")
    plan = qgemv.QGemv(enc)
    assert np.array_equal(plan.debug_unpack().cpu().numpy(), enc["codes"])
    check_y(run_b1(torch, plan, x16), enc, x16)
    plan.close()


@pytest.mark.parametrize("name,M,K,budget", [("attn7b_u3", 64, 4096, None), ("tiny_u4", 48, 512, None),
                                             ("tiny_u4", 40, 256, "all")])
def test_small_ssqr(torch, name, M, K, budget):
    """Encodings from the SSQR grid search (overflows of shrunk grids to the
    sparse part); 'all' makes every nonzero weight an outlier."""
    wl = WORKLOADS[name]
    W, _ = make_weights(wl, 0, M, K)
    M_, K_ = W.shape
    n = M_ * K_ if budget == "all" else outlier_count(wl, M_, K_)
    enc = encode.encode(W, wl.bits, "uniform", n, 16, pick="ssqr")
    x16 = make_x(wl, 1, K_, 0, M_)
    _say(f"[gpu] ssqr {name} M={M_} K={K_} alpha={enc['alpha']:.6f} nnz={enc['row_ptr'][-1]}")
    plan = qgemv.QGemv(enc)
    assert np.array_equal(plan.debug_unpack().cpu().numpy(), enc["codes"])
    check_y(run_b1(torch, plan, x16), enc, x16)
    xb = make_x(wl, 8, K_, 0, M_)
    check_y(run_bn(torch, plan, xb), enc, xb)
    plan.close()


def _custom(fmt, bits, M, K, row_nnz, seed=0):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(M, K)).astype(np.uint8)
    f = {"M": M, "K": K, "bits": bits, "fmt": fmt, "group": 16, "codes": codes,
         "codes_packed": pack.pack_bitstream(codes, bits)}
    if fmt == "uniform":
        f["scales"] = rng.uniform(1e-3, 3e-2, size=(M, K // 16)).astype(np.float16)
        f["zeros"] = rng.integers(0, 1 << bits, size=(M, K // 16)).astype(np.float16)
    elif fmt == "bpdq":
        f["group"] = 32
        f["coefs"] = (rng.standard_normal((M, K // 32, bits + 1)) * 0.03).astype(np.float16)
    else:
        f["lut"] = np.sort(rng.standard_normal((M, 1 << bits)) * 0.05, axis=1).astype(np.float16)
    rows, cols = [], []
    for i, n in enumerate(row_nnz):
        c = np.sort(rng.choice(K, size=n, replace=False))
        rows.append(np.full(n, i)); cols.append(c)
    rows = np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)
    cols = np.concatenate(cols).astype(np.int64) if cols else np.zeros(0, np.int64)
    vals = rng.uniform(-2.5, 2.5, size=len(rows))
    f["row_ptr"], f["col_idx"], f["values"] = csr_from_positions(M, rows, cols, vals)
    return f


@pytest.mark.parametrize("fmt,bits", [("uniform", 3), ("uniform", 4), ("lut", 3), ("lut", 4), ("bpdq", 3)])
def test_edge_cases(torch, fmt, bits):
    cases = {
        "no_outliers": _custom(fmt, bits, 70, 2048, [0] * 70, seed=1),
        "single_row": _custom(fmt, bits, 1, 4096, [5], seed=2),
        "k32": _custom(fmt, bits, 300, 32, [1] * 300, seed=3),
        "dense_csr_rows": _custom(fmt, bits, 9, 4096, [0, 700, 64, 65, 128, 320, 321, 1, 4096], seed=4),
        "max_k": _custom(fmt, bits, 5, 16384, [3, 0, 500, 7, 16384], seed=5),
    }
    for label, f in cases.items():
        _say(f"[gpu] edge {fmt}{bits} {label} M={f['M']} K={f['K']} nnz={f['row_ptr'][-1]}")
        x16 = np.random.default_rng(9).standard_normal((1, f["K"])).astype(np.float16)
        plan = qgemv.QGemv(f)
        codes = plan.debug_unpack().cpu().numpy()
        assert np.array_equal(codes, f["codes"]), label
        y = run_b1(torch, plan, x16)
        check_y(y, f, x16)
        plan.close()


def _rows_of(f, rng, extra=()):
    M = f["M"]
    nnz_row = np.diff(f["row_ptr"])
    heavy = np.argsort(-nnz_row, kind="stable")[:32]
    pick = rng.choice(M, size=min(M, 1024), replace=False)
    return np.unique(np.concatenate([[0, 1, M - 2, M - 1], heavy, pick, np.asarray(extra, np.int64)]))


@pytest.mark.parametrize("fmt,bits", [("lut", 4), ("lut", 3), ("uniform", 3), ("uniform", 4), ("bpdq", 3)])
@pytest.mark.parametrize("label,M,K,heavy", [
    ("tw8_ragged", 32768 - 5, 256, 0),      # 8 tiles per workgroup (two LUT-4 table regions), short last tile
    ("tw5", 16 * 256 * 5 - 3, 384, 0),      # 5 tiles: the second LUT-4 region holds one tile
    ("tw3_tw4", 16 * (256 * 3 + 100), 512, 0),  # 3 or 4 tiles per workgroup
    ("csr_heavy", 16 * 256 * 5, 4096, 1000),  # 40 rows of 1000 outliers in workgroup 0 (past any LDS copy)
])
def test_b1_multi_tile_workgroups(torch, fmt, bits, label, M, K, heavy):
    """Batch-1 shapes whose workgroups hold several tiles (the pair-table kernel
    for LUT-4 codes, the streaming kernel for the others)."""
    rng = np.random.default_rng(21)
    row_nnz = [int(v) for v in rng.integers(0, 4, size=M)]
    row_nnz[7] = K  # a full row
    for r in range(40):
        row_nnz[16 + r] = heavy if heavy else row_nnz[16 + r]
    f = _custom(fmt, bits, M, K, row_nnz, seed=11)
    _say(f"[gpu] b1 multi-tile {fmt}{bits} {label} M={M} K={K} nnz={f['row_ptr'][-1]}")
    x16 = np.random.default_rng(12).standard_normal((1, K)).astype(np.float16)
    plan = qgemv.QGemv(f)
    y1 = run_b1(torch, plan, x16)
    assert np.all(np.isfinite(y1)), "output not fully written"
    check_y(y1, f, x16, _rows_of(f, rng, extra=range(0, min(M, 160))))
    y2 = run_b1(torch, plan, x16)
    assert np.array_equal(y1, y2), "not bitwise deterministic"
    plan.close()


def test_zero_x_gives_zero_y(torch):
    f = _custom("lut", 4, 50, 4096, [10] * 50)
    plan = qgemv.QGemv(f)
    y = run_b1(torch, plan, np.zeros((1, 4096), np.float16))
    assert np.all(y == 0.0)


def test_run_argument_errors(torch):
    f = _custom("uniform", 4, 8, 64, [1] * 8)
    plan = qgemv.QGemv(f)
    x = torch.zeros((1, 64), dtype=torch.float16, device="cuda")
    y = torch.zeros((1, 8), dtype=torch.float32, device="cuda")
    L = qgemv.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.qgemv_run(plan._h, x.data_ptr() + 2, y.data_ptr(), 1, s) == -1
    assert L.qgemv_run(plan._h, x.data_ptr(), y.data_ptr(), 3, s) == -3
    # a descriptor that does not match the blob is refused at create time
    g = dict(f)
    g["row_ptr"] = f["row_ptr"].copy()
    g["nnz"] = int(f["row_ptr"][-1]) + 5
    import ctypes
    desc, keep = qgemv.make_weights(g)
    h = ctypes.c_void_p(0)
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(desc), plan.blob.data_ptr(), plan.blob_bytes) == -5
    plan.close()


def test_side_stream(torch):
    enc, x16 = oracle_case("mlp7b_lut3", 64, 4096)
    plan = qgemv.QGemv(enc)
    st = torch.cuda.Stream()
    x = torch.from_numpy(x16[:1].copy()).cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        y = plan.run(x)
    st.synchronize()
    check_y(y.cpu().numpy().astype(np.float64), enc, x16)


# ---- batch 8 / 16 (MFMA path) ------------------------------------------------

BATCHED_SMALL = [
    ("tiny_u4", None, None, 16),
    ("attn7b_u3", 200, 2080, 16),
    ("mlp7b_lut3", 33, 4128, 8),
    ("mlp70b_lut4", 24, 8192, 8),
    ("mlp70b_lut4", 40, 2080, 16),
    ("block7b_u3", 96, 11008, 16),
    ("mlp7b_bpdq3", 64, 4096, 8),
    ("mlp7b_bpdq3", 33, 2112, 16),
]


@pytest.mark.parametrize("name,M,K,B", BATCHED_SMALL)
def test_batched_oracle_encoded(torch, name, M, K, B):
    enc, _ = oracle_case(name, M, K)
    wl = WORKLOADS[name]
    x16 = make_x(wl, B, enc["K"], 0, enc["M"])
    _say(f"[gpu] batched {name} B={B} M={enc['M']} K={enc['K']} nnz={enc['row_ptr'][-1]}")
    plan = qgemv.QGemv(enc)
    y1 = run_bn(torch, plan, x16)
    check_y(y1, enc, x16)
    y2 = run_bn(torch, plan, x16)
    assert np.array_equal(y1, y2), "not bitwise deterministic"
    plan.close()


@pytest.mark.parametrize("fmt,bits", [("uniform", 3), ("uniform", 4), ("lut", 3), ("lut", 4), ("bpdq", 3)])
@pytest.mark.parametrize("B", [8, 16])
def test_batched_edge_cases(torch, fmt, bits, B):
    cases = {
        "no_outliers": _custom(fmt, bits, 70, 2048, [0] * 70, seed=1),
        "single_row": _custom(fmt, bits, 1, 4096, [5], seed=2),
        "k32": _custom(fmt, bits, 300, 32, [1] * 300, seed=3),
        "dense_csr_rows": _custom(fmt, bits, 9, 4096, [0, 700, 64, 65, 128, 320, 321, 1, 4096], seed=4),
        "max_k": _custom(fmt, bits, 5, 16384, [3, 0, 500, 7, 16384], seed=5),
        # over 256 tiles, so workgroups own two or three tiles (x resident in LDS)
        "multi_tile": _custom(fmt, bits, 8208, 384, [i % 6 for i in range(8208)], seed=6),
        # the first workgroup's outliers exceed what its LDS holds
        "csr_past_lds": _custom(fmt, bits, 4112, 1024, [1024] * 40 + [i % 4 for i in range(4072)], seed=7),
    }
    for label, f in cases.items():
        _say(f"[gpu] batched edge {fmt}{bits} B={B} {label} M={f['M']} K={f['K']} nnz={f['row_ptr'][-1]}")
        x16 = np.random.default_rng(9).standard_normal((B, f["K"])).astype(np.float16)
        plan = qgemv.QGemv(f)
        y = run_bn(torch, plan, x16)
        check_y(y, f, x16)
        plan.close()


def test_batched_rows_match_single(torch):
    """Each batch row of a batched run meets the tolerance of, and stays close to, its own batch-1 run."""
    enc, _ = oracle_case("mlp70b_lut4", 40, 2080)
    x16 = make_x(WORKLOADS["mlp70b_lut4"], 8, enc["K"], 0, enc["M"])
    plan = qgemv.QGemv(enc)
    yb = run_bn(torch, plan, x16)
    for b in range(8):
        y1 = run_b1(torch, plan, x16[b:b + 1])
        check_y(y1, enc, x16[b:b + 1])
        _, A = gemv.gemv_rows(enc, x16[b:b + 1])
        assert np.all(np.abs(yb[b] - y1[0]) <= 2e-4 * A[0] + 2e-6)
    plan.close()


# ---------------------------------------------------------------------------
# HPTQ: prefix-coded integers on one grid (batch 1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,bpw", [(64, 1024, 3.125), (33, 2048, 3.125), (21, 512, 2.5), (300, 256, 4.0)])
def test_hptq_oracle_encoded(torch, M, K, bpw):
    from oracle import hptq
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, M, K)
    enc = hptq.encode(W, 128, bpw)
    x16 = make_x(wl, 1, K, 0, M)
    _say(f"[gpu] hptq M={M} K={K} bpw={enc['row_bits'][-1] / W.size:.3f} nsym={len(enc['huff_sym'])} "
         f"maxlen={enc['huff_len'].max()}")
    plan = qgemv.QGemv(enc)
    y1 = run_b1(torch, plan, x16)
    y_ref, A = hptq.gemv(enc, x16)
    assert np.all(np.isfinite(y1)), "output not fully written"
    ok, worst = gemv.within_tolerance(y1, y_ref, A)
    assert ok, f"tolerance exceeded: worst {worst:.3f}"
    y2 = run_b1(torch, plan, x16)
    assert np.array_equal(y1, y2), "not bitwise deterministic"
    for B in (8, 16):  # x from L2, one MFMA column per batch row
        xb = make_x(wl, B, K, 0, M)
        yb = run_bn(torch, plan, xb)
        yr, Ab = hptq.gemv(enc, xb)
        ok, worst = gemv.within_tolerance(yb, yr, Ab)
        assert ok, f"batch {B}: tolerance exceeded: worst {worst:.3f}"
        assert np.array_equal(yb, run_bn(torch, plan, xb)), "batched run not bitwise deterministic"
        y1b = run_b1(torch, plan, xb[B - 1:B])
        assert np.all(np.abs(yb[B - 1] - y1b[0]) <= 2e-4 * Ab[B - 1] + 2e-6)
    plan.close()


def test_hptq_full_size_sampled(torch):
    f = format_case("mlp7b_hptq")
    M, K = f["M"], f["K"]
    _say(f"[gpu] hptq full M={M} K={K} bits={f['row_bits'][-1]}")
    x16 = make_x("mlp7b_hptq", 1, K, 0, M)
    plan = qgemv.QGemv(f)
    y = run_b1(torch, plan, x16)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], rng.choice(M, size=160, replace=False)]))
    check_y(y, dict(f, fmt="hptq"), x16, rows)
    xb = make_x("mlp7b_hptq", 16, K, 0, M)
    yb = run_bn(torch, plan, xb)
    check_y(yb, dict(f, fmt="hptq"), xb, rows)
    plan.close()


def _hptq_custom(M, K, sym, ln, p_zero, seed):
    """An HPTQ encoding with a given code: integers drawn from the code's
    alphabet (0 with probability p_zero), steps U(0.5, 1.5)/64."""
    from oracle import hptq
    rng = np.random.default_rng(seed)
    sym = np.asarray(sym, np.int64)
    ln = np.asarray(ln, np.int64)
    s_, l_, codes = hptq.canonical_code(sym, ln)
    nz = s_[s_ != 0]
    q = np.where(rng.random((M, K)) < p_zero, 0, rng.choice(nz, size=(M, K)))
    stream, row_bits = hptq.encode_stream(q, s_, l_, codes)
    scales = (rng.uniform(0.5, 1.5, size=(M, K // 128)) / 64).astype(np.float16)
    return {"M": M, "K": K, "fmt": "hptq", "group": 128, "scales": scales, "q": q, "huff_sym": s_.astype(np.int16),
            "huff_len": l_.astype(np.uint8), "huff_code": codes, "stream": stream, "row_bits": row_bits,
            "row_ptr": np.zeros(M + 1, np.int32), "col_idx": np.zeros(0, np.int32), "values": np.zeros(0, np.float16)}


def _hptq_lds_path(blob, K):
    """(second-level tables used, blocks decoded side by side) as the launcher chooses them at batch 1."""
    h = blob[:256].view(np.int32)
    nsym, hmaxw, nsub, tiles, nkb = int(h[36]), int(h[38]), int(h[39]), int(h[7]), int(h[23])
    tw = -(-tiles // min(tiles, 256))
    bufw = (hmaxw + 20 + 3) // 4 * 4
    static = 256 * 64 * 4 + 64
    for sub in (True, False):
        if sub and nsub > 64:
            continue
        aux = 256 * nsub * 4 if sub else ((nsym + 1) // 2 + 3) // 4 * 4 * 4
        fixed = K * 2 + aux + (tw + 15) * 64 + ((tw * nkb + 4) & ~3) * 4
        for g in (3, 2, 1):
            if static + fixed + 16 * g * bufw * 4 <= 160 * 1024:
                return sub, g
    return None


# 0 -> '0'; 4000 integers +-1..+-2000 of 13 bits: 125 eight-bit prefixes of long codewords
_CODE13 = ([0] + [v for a in range(1, 2001) for v in (-a, a)], [1] + [13] * 4000)
# 0 -> '0'; 2048 integers +-1..+-1024 of 16 bits: 8 prefixes
_CODE16 = ([0] + [v for a in range(1, 1025) for v in (-a, a)], [1] + [16] * 2048)


@pytest.mark.parametrize("code,p_zero,M,K,path", [
    (_CODE13, 0.85, 40, 512, (False, 3)),   # canonical search, three blocks side by side
    (_CODE13, 0.10, 24, 512, (False, 1)),   # canonical search, large blocks: one at a time
    (_CODE16, 0.55, 24, 512, (True, 2)),    # second-level tables, blocks of ~7.8 bits per weight: two
    (_CODE16, 0.10, 24, 512, (True, 1)),    # second-level tables, large blocks
])
def test_hptq_fallback_paths(torch, code, p_zero, M, K, path):
    from oracle import hptq
    enc = _hptq_custom(M, K, *code, p_zero, seed=M)
    blob = qgemv.repack(enc)
    assert _hptq_lds_path(blob, K) == path
    _say(f"[gpu] hptq path={path} M={M} K={K} bits/weight={enc['row_bits'][-1] / (M * K):.2f}")
    x16 = make_x(WORKLOADS["mlp7b_lut3"], 1, K, 0, M)
    plan = qgemv.QGemv(enc)
    y1 = run_b1(torch, plan, x16)
    y_ref, A = hptq.gemv(enc, x16)
    ok, worst = gemv.within_tolerance(y1, y_ref, A)
    assert ok, f"tolerance exceeded: worst {worst:.3f}"
    xb = make_x(WORKLOADS["mlp7b_lut3"], 8, K, 0, M)
    yb = run_bn(torch, plan, xb)
    yr, Ab = hptq.gemv(enc, xb)
    ok, worst = gemv.within_tolerance(yb, yr, Ab)
    assert ok, f"batch 8: tolerance exceeded: worst {worst:.3f}"
    plan.close()


@pytest.mark.parametrize("M,K", [(5, 256), (1, 128)])
def test_hptq_single_integer(torch, M, K):
    """An all-zero matrix: one integer, a one-bit code, only the filler second-level table; y is exactly 0."""
    from oracle import hptq
    enc = hptq.encode(np.zeros((M, K), np.float16), 128, 3.125)
    assert len(enc["huff_sym"]) == 1 and int(enc["huff_len"][0]) == 1
    blob = qgemv.repack(enc)
    assert int(blob[:256].view(np.int32)[39]) == 1
    _say(f"[gpu] hptq single integer M={M} K={K}")
    x16 = make_x(WORKLOADS["mlp7b_lut3"], 1, K, 0, M)
    plan = qgemv.QGemv(enc)
    y1 = run_b1(torch, plan, x16)
    assert np.array_equal(y1, np.zeros_like(y1))
    plan.close()


def test_hptq_create_rejects_inconsistent_headers(torch):
    """qgemv_create checks the blob's HPTQ fields it cannot derive from the shape."""
    from oracle import hptq
    W, _ = make_weights(WORKLOADS["mlp7b_lut3"], 0, 20, 256)
    enc = hptq.encode(W, 128, 3.125)
    good = qgemv.repack(enc)
    plan = qgemv.QGemv(enc, blob=good)  # the unmodified blob binds
    plan.close()
    for field, value in ((38, 6), (38, 1 << 20), (39, 0), (39, 1 << 20)):  # hmaxw not a multiple of 4 / too big; hsub
        bad = good.copy()
        bad[:256].view(np.int32)[field] = value
        _say(f"[gpu] hptq header field {field} = {value}")
        with pytest.raises(qgemv.QgemvError) as err:
            qgemv.QGemv(enc, blob=bad)
        assert err.value.status == -5  # QGEMV_ERR_SIZE


@pytest.mark.gpu
def test_read_probe_reads_every_byte(torch):
    """The read probe used for the measured ceiling: sink[t] must be the XOR of
    the dwords of pieces t, t + T, ... (a ragged size, not a multiple of T)."""
    from dense_sparse_bit_amd import qgemv
    rng = np.random.default_rng(11)
    nbytes = 3 * (1 << 20) + 48
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    for words in (256, 1024 * 256):
        sink = torch.zeros(words, dtype=torch.int32, device="cuda")
        qgemv.read_probe(src, sink)
        torch.cuda.synchronize()
        T = min(1024, words // 256) * 256
        piece = np.bitwise_xor.reduce(host.view(np.uint32).reshape(-1, 4), axis=1)
        want = np.zeros(T, np.uint32)
        for t in range(min(T, len(piece))):
            want[t] = np.bitwise_xor.reduce(piece[t::T])
        got = sink.cpu().numpy().view(np.uint32)[:T]
        assert np.array_equal(got, want)
    bad = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(qgemv.QgemvError):
        qgemv.read_probe(src[:40], bad)  # 40 bytes: not a multiple of 16
    with pytest.raises(qgemv.QgemvError):
        qgemv.read_probe(src, bad[:128])  # fewer than 256 sink words
