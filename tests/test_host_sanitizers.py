"""The repacker and its host inverse under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

qgemv_host.cpp is compiled with g++ -fsanitize=address,undefined together
with tests/native/host_sanitize_driver.cpp, which gives every input array a
heap block of exactly its documented length, calls qgemv_packed_size,
qgemv_repack (also one byte short) and qgemv_unpack_host (also on every
header word set to other values, and on a truncated blob).  A sanitizer
report fails the test; the blob must equal the normal library's byte for
byte and the codes must come back.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from dense_sparse_bit_amd import qgemv
from oracle import hptq, pack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "native", "host_sanitize_driver.cpp")
HOST = os.path.join(ROOT, "dense_sparse_bit_amd", "csrc", "qgemv_host.cpp")
ORDER = ("codes", "scales", "zeros", "lut", "row_ptr", "col_idx", "values", "coefs", "huff_len", "huff_sym",
         "row_bits")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("asan") / "host_sanitize_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Wno-unused-function", DRIVER, HOST, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _write_case(path, w):
    fmt = qgemv.FMT[w["fmt"]]
    hp = fmt == qgemv.FMT["hptq"]
    arrays = {
        "codes": w["stream"] if hp else w["codes_packed"],
        "scales": w.get("scales"), "zeros": w.get("zeros"), "lut": w.get("lut"),
        "row_ptr": w["row_ptr"], "col_idx": w.get("col_idx"), "values": w.get("values"), "coefs": w.get("coefs"),
        "huff_len": w.get("huff_len") if hp else None, "huff_sym": w.get("huff_sym") if hp else None,
        "row_bits": w.get("row_bits") if hp else None,
    }
    dtypes = {"codes": np.uint8, "scales": np.float16, "zeros": np.float16, "lut": np.float16, "row_ptr": np.int32,
              "col_idx": np.int32, "values": np.float16, "coefs": np.float16, "huff_len": np.uint8,
              "huff_sym": np.int16, "row_bits": np.int64}
    nnz = int(np.asarray(w["row_ptr"])[-1])
    head = [w["M"], w["K"], 0 if hp else w["bits"], fmt, int(w.get("group", 16) or 16), nnz,
            len(w["huff_sym"]) if hp else 0, 0]
    with open(path, "wb") as f:
        f.write(np.asarray(head, np.int64).tobytes())
        for k in ORDER:
            a = arrays[k]
            raw = b"" if a is None or np.asarray(a).size == 0 else np.ascontiguousarray(a, dtypes[k]).tobytes()
            f.write(np.int64(len(raw)).tobytes())
            f.write(raw)


def _run(driver, tmp_path, w, name):
    case, blob, codes = (str(tmp_path / f"{name}.{e}") for e in ("case", "blob", "codes"))
    _write_case(case, w)
    r = subprocess.run([driver, case, blob, codes], capture_output=True, text=True, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in report and "runtime error" not in report, report
    status = {}
    for line in r.stdout.splitlines():
        k, *v = line.split()
        status[k] = [int(t) for t in v]
    return status, blob, codes


def _canonical(fmt, bits, M, K, seed, nnz_rows=(0, 1, 3), group=32, full_row=None):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(M, K)).astype(np.uint8)
    w = {"M": M, "K": K, "bits": bits, "fmt": fmt,
         "group": 16 if fmt == "uniform" else group if fmt == "bpdq" else 0,
         "codes": codes, "codes_packed": pack.pack_bitstream(codes, bits)}
    if fmt == "uniform":
        w["scales"] = rng.uniform(1e-3, 2e-2, size=(M, K // 16)).astype(np.float16)
        w["zeros"] = rng.integers(0, 1 << bits, size=(M, K // 16)).astype(np.float16)
    elif fmt == "bpdq":
        w["coefs"] = (rng.standard_normal((M, K // group, bits + 1)) * 0.03).astype(np.float16)
    else:
        w["lut"] = np.sort(rng.standard_normal((M, 1 << bits)) * 0.05, axis=1).astype(np.float16)
    cols = []
    for i in range(M):
        n = K if i == full_row else int(rng.choice(nnz_rows))
        cols.append(np.sort(rng.choice(K, size=min(K, n), replace=False)))
    w["row_ptr"] = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    w["col_idx"] = np.concatenate(cols).astype(np.int32)
    w["values"] = rng.uniform(-2, 2, size=len(w["col_idx"])).astype(np.float16)
    return w


CASES = [(f, b, M, K) for f, b in (("uniform", 3), ("uniform", 4), ("lut", 3), ("lut", 4), ("bpdq", 3))
         for M, K in ((1, 32), (17, 160), (40, 2080), (3, 16384))]


@pytest.mark.parametrize("fmt,bits,M,K", CASES)
def test_repack_and_unpack_under_sanitizers(driver, tmp_path, fmt, bits, M, K):
    w = _canonical(fmt, bits, M, K, seed=M * 7 + K + bits, full_row=M - 1)
    st, blob, codes = _run(driver, tmp_path, w, "c")
    assert st["packed_size"][0] == 0 and st["repack"] == [0] and st["repack_short"] == [-5]
    assert st["unpack"] == [0] and st["unpack_truncated"] == [-5]
    assert st["header_fuzz"][1] > 0
    assert np.array_equal(np.fromfile(blob, np.uint8), qgemv.repack(w))
    assert np.array_equal(np.fromfile(codes, np.uint8).reshape(M, K), w["codes"])


def _hptq_case(M, K, sym, ln, p_zero, seed):
    rng = np.random.default_rng(seed)
    s_, l_, cw = hptq.canonical_code(np.asarray(sym, np.int64), np.asarray(ln, np.int64))
    nz = s_[s_ != 0] if np.any(s_ != 0) else s_
    q = np.where(rng.random((M, K)) < p_zero, s_[0] if 0 not in s_ else 0, rng.choice(nz, size=(M, K)))
    stream, row_bits = hptq.encode_stream(q, s_, l_, cw)
    return {"M": M, "K": K, "fmt": "hptq", "group": 128,
            "scales": (rng.uniform(0.5, 1.5, size=(M, K // 128)) / 64).astype(np.float16),
            "huff_sym": s_.astype(np.int16), "huff_len": l_.astype(np.uint8), "stream": stream,
            "row_bits": row_bits, "row_ptr": np.zeros(M + 1, np.int32), "col_idx": np.zeros(0, np.int32),
            "values": np.zeros(0, np.float16)}


HPTQ_CODES = {
    "short": ([0, -1, 1, -2, 2], [1, 3, 3, 3, 3]),
    "long13": ([0] + [v for a in range(1, 201) for v in (-a, a)], [1] + [12] * 400),
    "long16": ([0] + [v for a in range(1, 1025) for v in (-a, a)], [1] + [16] * 2048),
    "single": ([0], [1]),
}


@pytest.mark.parametrize("code", sorted(HPTQ_CODES))
@pytest.mark.parametrize("M,K", [(3, 128), (21, 512)])
def test_hptq_repack_under_sanitizers(driver, tmp_path, code, M, K):
    w = _hptq_case(M, K, *HPTQ_CODES[code], 0.6, seed=M + K)
    st, blob, _ = _run(driver, tmp_path, w, "h")
    assert st["packed_size"][0] == 0 and st["repack"] == [0] and st["repack_short"] == [-5]
    assert np.array_equal(np.fromfile(blob, np.uint8), qgemv.repack(w))


def _bad_cases():
    w = _canonical("lut", 4, 6, 64, seed=3, nnz_rows=(2,))
    out = []
    b = dict(w); b["col_idx"] = w["col_idx"].copy(); b["col_idx"][3] = 64
    out.append(("col_out_of_range", b))
    b = dict(w); b["col_idx"] = w["col_idx"].copy(); b["col_idx"][1] = b["col_idx"][0]
    out.append(("col_not_ascending", b))
    b = dict(w); b["row_ptr"] = w["row_ptr"].copy(); b["row_ptr"][2], b["row_ptr"][3] = 6, 3
    out.append(("row_ptr_decreasing", b))
    b = dict(w); b["lut"] = w["lut"].copy(); b["lut"][1, 1] = np.inf
    out.append(("lut_not_finite", b))
    h = _hptq_case(4, 256, *HPTQ_CODES["short"], 0.5, seed=1)
    b = dict(h); b["row_bits"] = h["row_bits"].copy(); b["row_bits"][2] += 1
    out.append(("hptq_row_bits_shifted", b))
    b = dict(h); b["huff_len"] = h["huff_len"].copy(); b["huff_len"][0] = 2  # Kraft sum 1/4 + 4/8 ... changes code
    out.append(("hptq_lengths_changed", b))
    b = dict(h); b["huff_len"] = np.array([1, 1, 3, 3, 3], np.uint8)  # Kraft sum above 1
    out.append(("hptq_kraft_above_one", b))
    b = dict(h); b["huff_sym"] = h["huff_sym"].copy(); b["huff_sym"][2] = b["huff_sym"][1]
    out.append(("hptq_duplicate_integer", b))
    return out


@pytest.mark.parametrize("label,w", _bad_cases(), ids=[c[0] for c in _bad_cases()])
def test_invalid_inputs_refused_under_sanitizers(driver, tmp_path, label, w):
    st, _, _ = _run(driver, tmp_path, w, "bad")
    assert st["packed_size"][0] < 0, label
