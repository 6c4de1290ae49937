"""Oracle decode and dense-and-sparse GEMV in fp64 -- test infrastructure only.

[SqLLM] "2. Dense-and-Sparse decomposition": W = W_dense + W_sparse, so
    y = W x = dequant(W_dense) x + W_sparse x.
[SpQR] "Le format de stockage sparse": W_sparse is held as CSR (values FP16,
col_idx, row_ptr).

`y[b, i] = sum_j d_ij x[b, j] + sum_{p in row i} r_p x[b, col_p]`, all in fp64
from the FP16 inputs.  The tolerance scale of every output is
`A[b, i] = sum_j |w_ij x[b, j]|`, where w = d + s is the weight the product
uses: the decoded dense part plus the CSR entry at (i, j), if any.  Where a
hole decodes to exactly 0 this equals sum_j |d_ij x_j| + sum_p |r_p x_col|;
where a dense value and a residual share a position it is the tighter of
the two.
"""

from __future__ import annotations

import numpy as np

from .pack import unpack_bitstream


def decode_rows(enc: dict, rows=None, codes: np.ndarray | None = None) -> np.ndarray:
    """Dense decoded weights d [len(rows), K] in fp64.

    Uniform ([SpQR] "Quantification d'un modèle", groupsize 16):
        d_ij = scale_{i,g(j)} * (q_ij - zero_{i,g(j)}),  g(j) = j // group
    LUT ([SqLLM] "Non-uniform quantization via Lloyd-Max optimisé"):
        d_ij = LUT_i[q_ij]
    BPDQ ([BPDQ] "1. Formulation de la Grille Variable"):
        d_ij = C0 + sum_t C_t * bit_(t-1)(q_ij), coefficients of (row i, group j // group)
    Codes are read from the packed bitstream unless given.
    """
    if enc["fmt"] == "hptq":
        # [Babai/GPTQ] "3. Applications Pratiques et Algorithmes", HPTQ: d = s * q from the prefix-coded stream
        from .hptq import decode_rows as hptq_rows
        return hptq_rows(enc, rows)
    M, K, bits = enc["M"], enc["K"], enc["bits"]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    if codes is None:
        codes = unpack_bitstream(np.asarray(enc["codes_packed"])[rows], bits, K)
    q = codes.astype(np.float64)
    if enc["fmt"] == "uniform":
        g = enc["group"]
        s = np.repeat(np.asarray(enc["scales"])[rows].astype(np.float64), g, axis=1)
        z = np.repeat(np.asarray(enc["zeros"])[rows].astype(np.float64), g, axis=1)
        return s * (q - z)
    if enc["fmt"] == "lut":
        lut = np.asarray(enc["lut"])[rows].astype(np.float64)
        return np.take_along_axis(lut, codes.astype(np.int64), axis=1)
    if enc["fmt"] == "bpdq":
        # [BPDQ] "1. Formulation de la Grille Variable": d = C0 + sum_i C_i * B_i,
        # coefficients per (row, group), plane i = bit i-1 of the code.
        g = enc["group"]
        C = np.repeat(np.asarray(enc["coefs"])[rows].astype(np.float64), g, axis=1)  # [R, K, bits+1]
        c = codes.astype(np.int64)
        d = C[:, :, 0].copy()
        for i in range(1, bits + 1):
            d += C[:, :, i] * ((c >> (i - 1)) & 1)
        return d
    raise ValueError(enc["fmt"])


def decode(enc: dict) -> np.ndarray:
    """All rows of the dense part, decoded from the unpacked codes if present."""
    return decode_rows(enc, None, enc.get("codes"))


def sparse_rows(enc: dict, rows) -> tuple:
    """(local row index, column, value as fp64) of the CSR entries of `rows`."""
    rp = np.asarray(enc["row_ptr"], dtype=np.int64)
    ci = np.asarray(enc["col_idx"], dtype=np.int64)
    va = np.asarray(enc["values"]).astype(np.float64)
    loc, col, val = [], [], []
    for li, i in enumerate(rows):
        a, b = rp[i], rp[i + 1]
        loc.append(np.full(b - a, li, dtype=np.int64))
        col.append(ci[a:b])
        val.append(va[a:b])
    if not loc:
        return np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0)
    return np.concatenate(loc), np.concatenate(col), np.concatenate(val)


def gemv_rows(enc: dict, X16: np.ndarray, rows=None, D: np.ndarray | None = None, scale: bool = True):
    """y and its tolerance scale A for the selected output rows.

    X16: activations [B, K] (FP16).  Returns (y [B, len(rows)], A [B, len(rows)]) in fp64;
    A is None when scale is False (y only).
    """
    M = enc["M"]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    x = np.asarray(X16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    if D is None:
        D = decode_rows(enc, rows)
    y = x @ D.T
    loc, col, val = sparse_rows(enc, rows)
    contrib = val[None, :] * x[:, col]            # [B, nnz_sel]
    for b in range(x.shape[0]):
        np.add.at(y[b], loc, contrib[b])
    return y, (tolerance_scale(x, D, loc, col, val) if scale else None)


def tolerance_scale(x: np.ndarray, D: np.ndarray, loc, col, val) -> np.ndarray:
    """A [B, R] = sum_j |w_ij x[b, j]| with w = D + the sparse entries (loc, col, val).

    x: fp64 [B, K]; D: decoded dense rows [R, K]; loc/col/val: the CSR entries
    of those rows (local row, column, fp64 value).
    """
    W = np.array(D, dtype=np.float64, copy=True)
    np.add.at(W, (np.asarray(loc, np.int64), np.asarray(col, np.int64)), val)
    return np.abs(x) @ np.abs(W).T


def gemv(enc: dict, X16: np.ndarray):
    """Full y [B, M] and A [B, M]."""
    return gemv_rows(enc, X16, None, decode(enc))


def sparse_dense(enc: dict) -> np.ndarray:
    """W_sparse as a dense fp64 [M, K] matrix (scatter of the CSR)."""
    M, K = enc["M"], enc["K"]
    S = np.zeros((M, K))
    loc, col, val = sparse_rows(enc, np.arange(M))
    np.add.at(S, (loc, col), val)
    return S


def within_tolerance(y_test, y_ref, A, rel=1e-4, abs_=1e-6):
    """The per-output acceptance test |y_test - y| <= rel * A + abs_; returns (ok, worst ratio)."""
    err = np.abs(np.asarray(y_test, dtype=np.float64) - y_ref)
    bound = rel * A + abs_
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = err / bound
    return bool(np.all(err <= bound)), float(ratio.max()) if ratio.size else 0.0
