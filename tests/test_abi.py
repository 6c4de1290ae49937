"""Host-side checks of the C ABI: exported symbols, validation, and the repacker.

No GPU is needed: only qgemv_packed_size / qgemv_repack / qgemv_unpack_host /
qgemv_error_string and argument checks that fail before any HIP call run here.
"""

import ctypes

import numpy as np
import pytest

from dense_sparse_bit_amd import qgemv
from oracle import encode, pack
from synth import WORKLOADS, make_weights, make_x, outlier_count


def test_library_exports_every_declared_symbol():
    L = qgemv.lib()
    names = qgemv.header_symbols()
    assert len(names) == 11
    for n in names:
        assert hasattr(L, n), n


def test_error_strings():
    L = qgemv.lib()
    for st in [0, -1, -2, -3, -4, -5, -6, 7]:
        s = L.qgemv_error_string(st)
        assert isinstance(s, bytes) and len(s) > 0
    assert L.qgemv_error_string(0) == b"ok"
    assert L.qgemv_last_hip_error() == 0


def _random_canonical(fmt, bits, M, K, nnz_per_row=3, seed=0, group=32):
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
    cols = [np.sort(rng.choice(K, size=min(K, nnz_per_row), replace=False)) for _ in range(M)]
    w["row_ptr"] = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    w["col_idx"] = np.concatenate(cols).astype(np.int32)
    w["values"] = rng.uniform(-2, 2, size=len(w["col_idx"])).astype(np.float16)
    return w


FORMATS = [("uniform", 3), ("uniform", 4), ("lut", 3), ("lut", 4), ("bpdq", 3)]


@pytest.mark.parametrize("fmt,bits", FORMATS)
@pytest.mark.parametrize("K", [32, 64, 2048, 2080, 4128, 11008])
def test_repack_roundtrip_random(fmt, bits, K):
    w = _random_canonical(fmt, bits, 5, K, seed=K + bits)
    blob = qgemv.repack(w)
    assert blob.size == qgemv.packed_size(w)
    assert blob.size % 256 == 0
    assert np.array_equal(qgemv.unpack_host(blob, 5, K), w["codes"])
    assert np.array_equal(qgemv.repack(w), blob)   # deterministic


@pytest.mark.parametrize("fmt,bits", FORMATS)
def test_repack_roundtrip_every_code_value_in_every_slot(fmt, bits):
    K = 32 * (1 << bits)
    codes = np.array([[(j + r) % (1 << bits) for j in range(K)] for r in range(1 << bits)], dtype=np.uint8)
    w = _random_canonical(fmt, bits, codes.shape[0], K)
    w["codes"], w["codes_packed"] = codes, pack.pack_bitstream(codes, bits)
    assert np.array_equal(qgemv.unpack_host(qgemv.repack(w), codes.shape[0], K), codes)


@pytest.mark.parametrize("name,M,K", [("tiny_u4", None, None), ("attn7b_u3", 40, 2080),
                                      ("mlp7b_lut3", 12, 4096), ("mlp70b_lut4", 6, 4128),
                                      ("mlp7b_bpdq3", 20, 1024)])
def test_repack_roundtrip_oracle_encoding(name, M, K):
    wl = WORKLOADS[name]
    W, planted = make_weights(wl, 0, M, K)
    M, K = W.shape
    x = make_x(wl, 1, K, 0, M)
    enc = encode.encode(W, wl.bits, wl.fmt, outlier_count(wl, M, K), wl.group or 16,
                        sens=x[0].astype(np.float64) ** 2)
    blob = qgemv.repack(enc)
    assert np.array_equal(qgemv.unpack_host(blob, M, K), enc["codes"])
    # header, row_ptr and entries sections
    hdr = blob[:256].view(np.uint32)
    assert hdr[0] == 0x564D4751 and hdr[2] == M and hdr[3] == K and hdr[4] == wl.bits
    off = blob[:256].view(np.uint64)
    nnz = int(blob[32:40].view(np.int64)[0])
    assert nnz == enc["row_ptr"][-1]
    off_rowptr, off_entries = int(off[7]), int(off[8])
    assert np.array_equal(blob[off_rowptr:off_rowptr + 4 * (M + 1)].view(np.int32), enc["row_ptr"])
    ent = blob[off_entries:off_entries + 4 * nnz].view(np.uint32)
    assert np.array_equal(ent & 0xFFFF, enc["col_idx"])
    assert np.array_equal((ent >> 16).astype(np.uint16), enc["values"].view(np.uint16))
    _check_block_outliers(blob, enc, M, K)


def _check_block_outliers(blob, w, M, K):
    """The outliers grouped by (tile, K-block) are the CSR outliers, each once, in row-then-column order."""
    off = blob[:256].view(np.uint64)
    off_boff, off_bent = int(off[12]), int(off[13])
    tiles, nkb = (M + 15) // 16, (K + 127) // 128
    nnz = int(w["row_ptr"][-1])
    boff = blob[off_boff:off_boff + 4 * (tiles * nkb + 1)].view(np.int32)
    bent = blob[off_bent:off_bent + 4 * nnz].view(np.uint32)
    assert boff[0] == 0 and boff[-1] == nnz and np.all(np.diff(boff) >= 0)
    rows = np.repeat(np.arange(M), np.diff(w["row_ptr"]))
    cols = np.asarray(w["col_idx"], dtype=np.int64)
    vals = np.asarray(w["values"]).view(np.uint16)
    blk = (rows // 16) * nkb + cols // 128
    order = np.lexsort((cols, rows, blk))
    assert np.array_equal(np.bincount(blk, minlength=tiles * nkb), np.diff(boff))
    exp = (cols[order] % 128) | ((rows[order] % 16) << 7) | (vals[order].astype(np.int64) << 16)
    assert np.array_equal(bent.astype(np.int64), exp)


def _status(w):
    try:
        qgemv.packed_size(w)
        return 0
    except qgemv.QgemvError as e:
        return e.status


def test_validation_errors():
    base = _random_canonical("uniform", 4, 4, 64)
    assert _status(base) == 0
    INV, CSR, UNS = -1, -2, -3

    def mod(**kw):
        w = dict(base)
        w.update(kw)
        return w
    assert _status(mod(bits=5)) == UNS
    assert _status(mod(bits=2)) == UNS
    assert _status(mod(fmt=7)) == UNS
    assert _status(mod(group=32)) == UNS
    assert _status(mod(K=48, codes_packed=base["codes_packed"])) == UNS
    assert _status(mod(M=0)) == INV
    assert _status(mod(codes_packed=None)) == INV
    rp = base["row_ptr"].copy(); rp[0] = 1
    assert _status(mod(row_ptr=rp, nnz=int(base["row_ptr"][-1]))) == CSR
    rp = base["row_ptr"].copy(); rp[2], rp[1] = rp[1], rp[2]
    assert _status(mod(row_ptr=rp)) == CSR
    ci = base["col_idx"].copy(); ci[0] = 64
    assert _status(mod(col_idx=ci)) == CSR
    ci = base["col_idx"].copy(); ci[1] = ci[0]
    assert _status(mod(col_idx=ci)) == CSR
    ci = base["col_idx"].copy(); ci[0] = -1
    assert _status(mod(col_idx=ci)) == CSR
    z = base["zeros"].copy(); z[0, 0] = 16
    assert _status(mod(zeros=z)) == INV
    z = base["zeros"].copy(); z[0, 0] = 1.5
    assert _status(mod(zeros=z)) == INV
    s = base["scales"].copy(); s[0, 0] = np.nan
    assert _status(mod(scales=s)) == INV
    v = base["values"].copy(); v[0] = np.inf
    assert _status(mod(values=v)) == INV
    lw = _random_canonical("lut", 3, 4, 64)
    lut = lw["lut"].copy(); lut[1, 2] = np.inf
    w = dict(lw); w["lut"] = lut
    assert _status(w) == INV
    w = dict(lw); w["lut"] = None
    assert _status(w) == INV
    big = _random_canonical("lut", 4, 1, 32)
    big["K"] = 16384 + 32
    assert _status(big) == UNS


def test_nnz_mismatch_and_small_buffers():
    w = _random_canonical("lut", 4, 3, 64)
    w2 = dict(w); w2["nnz"] = int(w["row_ptr"][-1]) + 1
    assert _status(w2) == -2
    s, keep = qgemv.make_weights(w)
    n = qgemv.packed_size(w)
    buf = np.zeros(n - 1, dtype=np.uint8)
    assert qgemv.lib().qgemv_repack(ctypes.byref(s), buf.ctypes.data, n - 1) == -5
    assert qgemv.lib().qgemv_repack(ctypes.byref(s), None, n) == -1
    assert qgemv.lib().qgemv_packed_size(None, None) == -1


def test_unpack_host_rejects_garbage():
    junk = np.zeros(512, dtype=np.uint8)
    out = np.zeros(16, dtype=np.uint8)
    assert qgemv.lib().qgemv_unpack_host(junk.ctypes.data, junk.size, out.ctypes.data, out.size) == -5
    assert qgemv.lib().qgemv_unpack_host(None, 0, out.ctypes.data, out.size) == -1
    w = _random_canonical("uniform", 3, 2, 64)
    blob = qgemv.repack(w)
    assert qgemv.lib().qgemv_unpack_host(blob.ctypes.data, blob.size - 256, out.ctypes.data, out.size) == -5


@pytest.mark.parametrize("fmt,bits", [("uniform", 3), ("lut", 4), ("bpdq", 3)])
def test_unpack_host_rejects_inconsistent_header_fields(fmt, bits):
    """A header whose fields are not the repacker's for its own shape is refused
    (bits = 16 would otherwise copy 64-byte chunks into a 16-byte buffer)."""
    w = _random_canonical(fmt, bits, 20, 256)
    blob = qgemv.repack(w)
    out = np.zeros((20, 256), dtype=np.uint8)
    L = qgemv.lib()
    assert L.qgemv_unpack_host(blob.ctypes.data, blob.size, out.ctypes.data, out.size) == 0
    assert np.array_equal(out, w["codes"])
    # int32 words of the header: 4 bits, 5 format, 6 group, 7 tiles, 10 off_codes, 20 block_bytes, 23 nkb
    for word, value in ((4, 16), (4, 5), (5, 7), (6, 48), (7, 3), (7, 1 << 30), (10, 1 << 28),
                        (20, 64 * 4 * 16), (23, 64), (2, 1 << 20)):
        bad = blob.copy()
        bad[:256].view(np.int32)[word] = value
        assert L.qgemv_unpack_host(bad.ctypes.data, bad.size, out.ctypes.data, out.size) == -5, (word, value)
    # an output buffer one byte short of M*K
    assert L.qgemv_unpack_host(blob.ctypes.data, blob.size, out.ctypes.data, out.size - 1) == -5


def test_run_and_create_argument_checks_need_no_gpu():
    L = qgemv.lib()
    assert L.qgemv_run(None, None, None, 1, None) == -1
    assert L.qgemv_run_noalloc(None, None, None, 1, None) == -1
    assert L.qgemv_debug_unpack(None, None, None) == -1
    assert L.qgemv_destroy(None) == 0
    h = ctypes.c_void_p(0)
    assert L.qgemv_create(ctypes.byref(h), None, None, 0) == -1
    w = _random_canonical("lut", 4, 3, 64)
    s, keep = qgemv.make_weights(w)
    # misaligned device pointer is rejected before any HIP call
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(s), ctypes.c_void_p(0x1001), 1 << 20) == -1
    # a blob smaller than the descriptor needs is rejected before any HIP call
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(s), ctypes.c_void_p(0x100000), 256) == -5



@pytest.mark.parametrize("group,K", [(32, 4128), (64, 4096), (128, 384), (64, 1088)])
def test_bpdq_coefficients_in_blob(group, K):
    """Per (tile, K-block) the blob holds [16 rows][128/group][4] FP16 coefficients,
    zero for padding rows and for groups past K."""
    M = 21
    w = _random_canonical("bpdq", 3, M, K, group=group, seed=group)
    blob = qgemv.repack(w)
    off = blob[:256].view(np.uint64)
    off_meta = int(off[6])  # header: magic/version, M/K, bits/format, group/tiles, nnz, off_codes, off_meta
    tiles, nkb, gpk = (M + 15) // 16, (K + 127) // 128, 128 // group
    meta = blob[off_meta:off_meta + tiles * nkb * 16 * gpk * 8].view(np.uint16).reshape(tiles, nkb, 16, gpk, 4)
    want = np.zeros((tiles * 16, nkb * gpk, 4), dtype=np.uint16)
    want[:M, :K // group] = w["coefs"].view(np.uint16)
    want = want.reshape(tiles, 16, nkb, gpk, 4).transpose(0, 2, 1, 3, 4)
    assert np.array_equal(meta, want)


def test_bpdq_validation():
    INV, UNS = -1, -3
    base = _random_canonical("bpdq", 3, 4, 256, group=64)
    assert _status(base) == 0
    for bad in ({"bits": 4}, {"group": 16}, {"group": 48}):
        w = dict(base); w.update(bad)
        if "bits" in bad:
            w["codes"] = np.zeros((4, 256), np.uint8); w["codes_packed"] = pack.pack_bitstream(w["codes"], 4)
        assert _status(w) == UNS, bad
    w = _random_canonical("bpdq", 3, 4, 96, group=64)  # K % group != 0
    assert _status(w) == UNS
    w = dict(base); w["coefs"] = None
    assert _status(w) == INV
    c = base["coefs"].copy(); c[1, 2, 3] = np.nan
    w = dict(base); w["coefs"] = c
    assert _status(w) == INV
    c = base["coefs"].copy(); c[0, 0] = [40000.0, 30000.0, 0.0, 0.0]  # a level beyond FP16 range
    w = dict(base); w["coefs"] = c
    assert _status(w) == UNS


# ---------------------------------------------------------------------------
# HPTQ blobs
# ---------------------------------------------------------------------------
def _hptq_enc(M=21, K=512, seed=0):
    from oracle import hptq
    wl = WORKLOADS["mlp7b_lut3"]
    W, _ = make_weights(wl, 0, M, K)
    return hptq.encode(W, 128, 3.125 + 0.25 * seed)


def _decode_hptq_blob(blob):
    """The blob's integers [M, K] and steps, read the way the table decoder reads them."""
    hdr32 = blob[:256].view(np.int32)
    off = blob[:256].view(np.uint64)
    M, K, tiles = int(hdr32[2]), int(hdr32[3]), int(hdr32[7])
    nkb = int(hdr32[23])
    off_codes, off_meta, off_hidx, off_hlane, off_htab, off_hsym = (int(off[i]) for i in (5, 6, 14, 15, 16, 17))
    nsym = int(hdr32[36])
    hidx = blob[off_hidx:off_hidx + 4 * (tiles * nkb + 1)].view(np.uint32)
    words = blob[off_codes:off_codes + 4 * int(hidx[-1]) + 8].view(np.uint32)
    words = np.concatenate([words, np.zeros(2, np.uint32)])
    hlane = blob[off_hlane:off_hlane + 2 * 64 * tiles * nkb].view(np.uint16)
    tbits = 8
    nt = 1 << tbits
    tab = blob[off_htab:off_htab + 4 * (nt + 68)].view(np.int32)
    first, count, offs = tab[nt:nt + 17], tab[nt + 17:nt + 34], tab[nt + 34:nt + 51]
    ljlim = tab[nt + 51:nt + 68]
    nsub = int(hdr32[39])
    nsub_e = 1 << (16 - tbits)
    sub = blob[off_htab + 4 * (nt + 68):off_htab + 4 * (nt + 68 + nsub_e * nsub)].view(np.int32)
    syms = blob[off_hsym:off_hsym + 2 * nsym].view(np.int16)
    q = np.zeros((tiles * 16, nkb * 128), dtype=np.int64)
    for blk in range(tiles * nkb):
        t, b = divmod(blk, nkb)
        base = int(hidx[blk]) * 32
        for l in range(64):
            if t * 16 + l % 16 >= M:
                continue
            p = base + int(hlane[blk * 64 + l])
            for j in range(32):
                w0, w1 = int(words[p >> 5]), int(words[(p >> 5) + 1])
                win = ((w0 << 32 | w1) >> (32 - (p & 31))) & 0xFFFFFFFF
                e = int(tab[win >> (32 - tbits)]) & 0xFFFFFFFF
                if e & 255:
                    ln = e & 255
                    v = np.array([e >> 16], np.uint16).view(np.float16)[0]
                    assert float(v) == int(v)
                    v = int(v)
                else:
                    # the length is the shortest whose left-justified end lies above the prefix
                    p16 = win >> 16
                    ln2 = next(l for l in range(tbits + 1, 17) if p16 < ljlim[l])
                    # and the second-level table of the 12-bit prefix gives it with its integer
                    e2 = int(sub[(e >> 16) + (p16 & (nsub_e - 1))]) & 0xFFFFFFFF
                    v2 = int(np.array([e2 >> 16], np.uint16).view(np.float16)[0])
                    for ln in range(tbits + 1, 17):
                        c = win >> (32 - ln)
                        if count[ln] and first[ln] <= c < first[ln] + count[ln]:
                            v = int(syms[offs[ln] + c - first[ln]])
                            break
                    else:
                        raise AssertionError("no codeword")
                    assert ln2 == ln and (e2 & 255) == ln and v2 == v
                q[t * 16 + l % 16, b * 128 + 32 * (l // 16) + j] = v
                p += ln
    steps = blob[off_meta:off_meta + 32 * tiles * nkb].view(np.uint16).reshape(tiles, nkb, 16)
    steps = steps.transpose(0, 2, 1).reshape(tiles * 16, nkb)
    return q[:M, :K], steps[:M]


@pytest.mark.parametrize("M,K,seed", [(21, 512, 0), (16, 128, 1), (5, 1024, 2)])
def test_hptq_blob_decodes_to_oracle_integers(M, K, seed):
    enc = _hptq_enc(M, K, seed)
    blob = qgemv.repack(enc)
    q, steps = _decode_hptq_blob(blob)
    assert np.array_equal(q, enc["q"])
    assert np.array_equal(steps, enc["scales"].view(np.uint16))


def test_hptq_validation():
    INV, UNS = -1, -3
    enc = _hptq_enc(4, 256)
    assert _status(enc) == 0
    bad = dict(enc); bad["row_bits"] = enc["row_bits"].copy(); bad["row_bits"][1] += 1
    assert _status(bad) == INV                      # a row that does not hold exactly K codewords
    bad = dict(enc); bad["huff_len"] = enc["huff_len"][::-1].copy()
    assert _status(bad) == INV                      # lengths not canonical
    bad = dict(enc); bad["huff_sym"] = enc["huff_sym"].copy(); bad["huff_sym"][0] = 4000
    assert _status(bad) == INV                      # integer beyond 2048
    bad = dict(enc); bad["group"] = 64
    assert _status(bad) == UNS
    bad = dict(enc); bad["K"] = 96
    assert _status(bad) == UNS
    s = enc["scales"].copy(); s[0, 0] = np.inf
    bad = dict(enc); bad["scales"] = s
    assert _status(bad) == INV
    blob = qgemv.repack(enc)
    out = np.zeros(4 * 256, np.uint8)
    assert qgemv.lib().qgemv_unpack_host(blob.ctypes.data, blob.size, out.ctypes.data, out.size) == UNS


def test_hptq_blob_long_codewords():
    """The storage-format inputs' code has 14- and 16-bit codewords: the blob's
    second-level tables and left-justified limits decode them to the integers
    the stream was written from."""
    from synth import make_format_inputs
    f = make_format_inputs("mlp7b_hptq", 0, 37, 1024)
    f.update(row_ptr=np.zeros(38, np.int32), col_idx=np.zeros(0, np.int32), values=np.zeros(0, np.float16))
    blob = qgemv.repack(dict(f, fmt="hptq"))
    assert int(blob[:256].view(np.int32)[39]) > 0  # second-level tables present
    q, steps = _decode_hptq_blob(blob)
    assert np.array_equal(q, f["q"])
    assert np.array_equal(steps, f["scales"].view(np.uint16))
