"""Oracle for HPTQ, Huffman-coded integers on one unconstrained grid -- test infrastructure only.

[Babai/GPTQ] "3. Applications Pratiques et Algorithmes", HPTQ: inliers and
outliers share one integer grid with no clipping; the integers are Huffman
coded, so the bit width follows the weights' distribution, within a
compression budget (the pages report 3.125 bits per weight as a sweet spot).

Readings taken where the page is silent:
  * grid: per (row, group of `group` columns along K) an FP16 step that
    follows the bulk of the group, s = fp16(alpha * median |w_group|) (the
    group's max |w| if the median is 0, s = 1 if the group is all zero, 2^-24
    if the product rounds to 0), so that an outlier takes a large integer
    instead of stretching the grid; q = rint(w / s) with no clipping;
    d = s * q.  There is no sparse part: the grid holds the outliers too;
  * code: one prefix code for the whole matrix over the integers that occur,
    with lengths from package-merge (the optimal prefix code whose lengths do
    not exceed max_len = 16, so that a table decoder has a bounded window);
    a lone symbol gets length 1;
  * canonical codewords: symbols sorted by (length, value); the first
    codeword of each length is (first of the previous length + its count) << 1;
  * stream: the codewords of row 0, then row 1, ..., each written most
    significant bit first into one bit sequence, packed into bytes most
    significant bit first; row_bits[i] is the first bit of row i and
    row_bits[M] the total;
  * budget: alpha is the smallest value in (0, alpha_max] (to 40 halvings)
    whose stream takes at most `bpw` bits per weight; coarser grids take fewer.
"""

from __future__ import annotations

import numpy as np

from .encode import f16

FP16_MIN_SUBNORMAL = 2.0 ** -24


# --------------------------------------------------------------------------
# Grid
# --------------------------------------------------------------------------
def grid(W16: np.ndarray, group: int, alpha: float):
    """Steps s [M, K/group] (FP16 values as fp64) and integers q [M, K] (int64)."""
    M, K = W16.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    w = W16.astype(np.float64).reshape(M, K // group, group)
    a = np.abs(w)
    med = np.median(a, axis=2)
    base = np.where(med > 0, med, a.max(axis=2))
    s = f16(np.where(base > 0, alpha * base, 1.0))
    s = np.where(s == 0.0, FP16_MIN_SUBNORMAL, s)
    q = np.rint(w / s[:, :, None]).astype(np.int64)
    return s, q.reshape(M, K)


# --------------------------------------------------------------------------
# Prefix code
# --------------------------------------------------------------------------
def package_merge_lengths(freq: np.ndarray, max_len: int) -> np.ndarray:
    """Optimal code lengths with none above max_len (package-merge).

    Items start as the symbols sorted by frequency (ties: lower index first).
    max_len - 1 times, adjacent pairs of the current list are packaged (their
    weights added) and merged with the original items by weight (original
    items first on ties); the first 2n - 2 items of the last list are kept,
    and a symbol's length is the number of kept items that contain it.
    """
    n = len(freq)
    if n == 1:
        return np.ones(1, dtype=np.int64)
    if (1 << max_len) < n:
        raise ValueError("max_len too small for the alphabet")
    order = sorted(range(n), key=lambda i: (freq[i], i))
    leaves = [(float(freq[i]), {i: 1}) for i in order]
    cur = list(leaves)
    for _ in range(max_len - 1):
        packages = []
        for a in range(0, len(cur) - 1, 2):
            wa, ca = cur[a]
            wb, cb = cur[a + 1]
            c = dict(ca)
            for k, v in cb.items():
                c[k] = c.get(k, 0) + v
            packages.append((wa + wb, c))
        merged, i, j = [], 0, 0
        while i < len(leaves) or j < len(packages):
            if j >= len(packages) or (i < len(leaves) and leaves[i][0] <= packages[j][0]):
                merged.append(leaves[i]); i += 1
            else:
                merged.append(packages[j]); j += 1
        cur = merged
    lengths = np.zeros(n, dtype=np.int64)
    for _, c in cur[:2 * n - 2]:
        for k, v in c.items():
            lengths[k] += v
    return lengths


def canonical_code(symbols: np.ndarray, lengths: np.ndarray):
    """Canonical codewords: returns (symbols, lengths, codes) sorted by (length, symbol)."""
    order = np.lexsort((symbols, lengths))
    sym, ln = symbols[order], lengths[order]
    codes = np.zeros(len(sym), dtype=np.int64)
    code, prev = 0, int(ln[0])
    for k in range(len(sym)):
        if k > 0:
            code = (code + 1) << (int(ln[k]) - prev)
            prev = int(ln[k])
        codes[k] = code
    return sym, ln, codes


def build_code(q: np.ndarray, max_len: int = 16):
    """The matrix's canonical prefix code over the integers in q."""
    values, counts = np.unique(q, return_counts=True)
    lengths = package_merge_lengths(counts.astype(np.float64), max_len)
    return canonical_code(values.astype(np.int64), lengths)


# --------------------------------------------------------------------------
# Stream
# --------------------------------------------------------------------------
def encode_stream(q: np.ndarray, sym, ln, codes):
    """Bytes of the stream (MSB-first) and row_bits [M+1]."""
    M, K = q.shape
    look = {int(s): (int(c), int(l)) for s, c, l in zip(sym, codes, ln)}
    bits = []
    row_bits = np.zeros(M + 1, dtype=np.int64)
    for i in range(M):
        row_bits[i] = len(bits)
        for v in q[i]:
            c, l = look[int(v)]
            bits.extend((c >> (l - 1 - t)) & 1 for t in range(l))
    row_bits[M] = len(bits)
    nbytes = (len(bits) + 7) // 8
    arr = np.zeros(nbytes * 8, dtype=np.uint8)
    arr[:len(bits)] = bits
    return np.packbits(arr), row_bits


def decode_stream(stream: np.ndarray, row_bits: np.ndarray, K: int, sym, ln, codes) -> np.ndarray:
    """Integers [M, K] read back from the stream, one bit at a time."""
    M = len(row_bits) - 1
    table = {(int(l), int(c)): int(s) for s, c, l in zip(sym, codes, ln)}
    bits = np.unpackbits(np.asarray(stream, dtype=np.uint8))
    q = np.zeros((M, K), dtype=np.int64)
    for i in range(M):
        p = int(row_bits[i])
        for j in range(K):
            c, l = 0, 0
            while (l, c) not in table:
                c = (c << 1) | int(bits[p]); p += 1; l += 1
                if l > 64:
                    raise ValueError("not a codeword")
            q[i, j] = table[(l, c)]
        if p != row_bits[i + 1]:
            raise ValueError("row length mismatch")
    return q


def stream_bits(q: np.ndarray, max_len: int = 16) -> int:
    sym, ln, codes = build_code(q, max_len)
    vals, cnt = np.unique(q, return_counts=True)
    total = 0
    look = {int(s): int(l) for s, l in zip(sym, ln)}
    for v, c in zip(vals, cnt):
        total += look[int(v)] * int(c)
    return total


# --------------------------------------------------------------------------
# Budget and the whole encoder
# --------------------------------------------------------------------------
def budget_alpha(W16: np.ndarray, group: int, bpw: float, alpha_max: float = 8.0, iters: int = 40,
                 max_len: int = 16) -> float:
    """Smallest alpha in (0, alpha_max] whose stream takes at most bpw bits per weight."""
    n = W16.size
    fits = lambda a: stream_bits(grid(W16, group, a)[1], max_len) <= bpw * n
    if not fits(alpha_max):
        return alpha_max
    lo, hi = 0.0, alpha_max
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if fits(mid):
            hi = mid
        else:
            lo = mid
    return hi


def encode(W16: np.ndarray, group: int = 128, bpw: float = 3.125, max_len: int = 16) -> dict:
    """HPTQ encoding of an FP16 matrix: steps, integers, prefix code and stream."""
    M, K = W16.shape
    alpha = budget_alpha(W16, group, bpw, max_len=max_len)
    s, q = grid(W16, group, alpha)
    sym, ln, codes = build_code(q, max_len)
    stream, row_bits = encode_stream(q, sym, ln, codes)
    return {"M": M, "K": K, "fmt": "hptq", "group": group, "alpha": alpha, "scales": s.astype(np.float16),
            "q": q, "huff_sym": sym, "huff_len": ln, "huff_code": codes, "stream": stream, "row_bits": row_bits,
            "max_len": max_len,
            "row_ptr": np.zeros(M + 1, dtype=np.int32), "col_idx": np.zeros(0, np.int32),
            "values": np.zeros(0, np.float16)}


def decode_rows(enc: dict, rows=None) -> np.ndarray:
    """d = s * q for the given rows, read from the stream row by row (canonical
    codewords rebuilt from the integers and lengths)."""
    M, K = enc["M"], enc["K"]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    sym, ln, codes = canonical_code(np.asarray(enc["huff_sym"], np.int64), np.asarray(enc["huff_len"], np.int64))
    rb = np.asarray(enc["row_bits"], np.int64)
    q = np.zeros((len(rows), K), dtype=np.int64)
    for k, i in enumerate(rows):
        q[k] = decode_stream(enc["stream"], rb[[i, i + 1]], K, sym, ln, codes)[0]
    s = np.repeat(np.asarray(enc["scales"])[rows].astype(np.float64), enc["group"], axis=1)
    return s * q


def decode(enc: dict) -> np.ndarray:
    """d = s * q, q read back from the stream."""
    q = decode_stream(enc["stream"], enc["row_bits"], enc["K"], enc["huff_sym"], enc["huff_len"], enc["huff_code"])
    s = np.repeat(np.asarray(enc["scales"]).astype(np.float64), enc["group"], axis=1)
    return s * q


def gemv(enc: dict, X16: np.ndarray, rows=None):
    """y and its tolerance scale A (rows optional), fp64.

    There is no sparse part, so A[b, i] = sum_j |d_ij x[b, j]| (the tolerance
    scale of the dense-and-sparse GEMV with an empty CSR).
    """
    from .gemv import tolerance_scale
    D = decode(enc) if rows is None else decode_rows(enc, rows)
    x = np.asarray(X16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    none = np.zeros(0, np.int64)
    return x @ D.T, tolerance_scale(x, D, none, none, np.zeros(0))
