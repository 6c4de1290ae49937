"""Seeded generators for the five GEMV workloads.

Every array is drawn from ``numpy.random.default_rng([wid, layer, stream, M, K])``
so that a (workload, layer, shape) triple always yields the same bits.  The
streams are: 0 bulk weights, 1 outlier positions, 2 outlier values and signs,
3 activations x, 4 synthetic format arrays.

The weight laws follow the workloads' descriptions: a Gaussian bulk (the
"distribution gaussienne" concentrated around zero on the page "SpQR
(Sparse-Quantized Representation)", section "Qu'est-ce qu'un poids outlier ?")
plus a small fraction of large-magnitude outliers (about 1 % on that page,
section "La solution SpQR : décomposition sparse + dense"; about 0.45 % on the
page "SqueezeLLM (Dense-and-Sparse Quantization)", section "Sélection des
outliers").  All weights are stored in FP16, as in that SpQR page's section
"Diagramme de la matrice sparse vs dense".

Nothing here quantizes, packs, decodes or multiplies.
"""

from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache

import numpy as np


@dataclass(frozen=True)
class Workload:
    wid: int            # numeric id used in the seed
    name: str           # short name, e.g. "mlp70b_lut4"
    title: str
    M: int              # output rows (out features)
    K: int              # input columns (in features)
    bits: int           # code width
    fmt: str            # "uniform" (group scale/zero), "lut" (per-row table) or "bpdq" (bit-plane coefficients)
    group: int          # group size along K for "uniform" and "bpdq", 0 for "lut"
    density: float      # outlier fraction of M*K
    sigma: float        # std of the Gaussian bulk
    law: str            # outlier placement law (see make_weights)
    batches: tuple      # batch sizes the workload is run at
    layers: tuple = ()  # ((layer_name, M, K), ...) for multi-layer workloads


WORKLOADS = {
    "tiny_u4": Workload(
        1, "tiny_u4",
        "512x512, 4-bit asymmetric uniform g16, top-1% |w| replaced by +-U(0.2,2.5)",
        512, 512, 4, "uniform", 16, 0.01, 0.02, "top_bulk", (1,)),
    "attn7b_u3": Workload(
        2, "attn7b_u3",
        "LLaMA-7B attention projection 4096x4096, 3-bit uniform g16, 0.5% Student-t(3)x0.1 outliers",
        4096, 4096, 3, "uniform", 16, 0.005, 0.02, "student_t_top", (1,)),
    "mlp7b_lut3": Workload(
        3, "mlp7b_lut3",
        "SqueezeLLM-style MLP up-proj 11008x4096, 3-bit per-row LUT-8, 0.45% outliers",
        11008, 4096, 3, "lut", 0, 0.0045, 0.02, "uniform_pos", (1,)),
    "mlp70b_lut4": Workload(
        4, "mlp70b_lut4",
        "70B-shaped MLP 28672x8192, 4-bit per-row LUT-16, 0.5% row-skewed outliers + 2 full columns",
        28672, 8192, 4, "lut", 0, 0.005, 0.015, "row_skewed", (1, 8)),
    "block7b_u3": Workload(
        5, "block7b_u3",
        "7B decoder block (q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008), 3-bit uniform g16, 1% outliers",
        4096, 4096, 3, "uniform", 16, 0.01, 0.02, "uniform_pos", (16,),
        (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
         ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))),
    "mlp7b_bpdq3": Workload(
        6, "mlp7b_bpdq3",
        "MLP up-proj 11008x4096, 3-bit BPDQ variable grid (4 FP16 coefficients per row and group of 64), 0.45% outliers",
        11008, 4096, 3, "bpdq", 64, 0.0045, 0.02, "uniform_pos", (1, 8)),
    "mlp7b_hptq": Workload(
        7, "mlp7b_hptq",
        "MLP up-proj 11008x4096, HPTQ: prefix-coded integers on one grid (FP16 step per row and group of 128), "
        "about 3.2 bits per weight, 0.45% outliers on the same grid",
        11008, 4096, 0, "hptq", 128, 0.0045, 0.02, "uniform_pos", (1,)),
}

# Synthetic prefix code for HPTQ storage-format inputs: integer length classes
# 0 -> 2 bits, +-1 -> 3, +-2..3 -> 4, +-4..7 -> 6, +-8..15 -> 8, ..., +-128..255 -> 16.
_HPTQ_CLASSES = [(0, 0, 2), (1, 1, 3), (2, 3, 4), (4, 7, 6), (8, 15, 8), (16, 31, 10), (32, 63, 12),
                 (64, 127, 14), (128, 255, 16)]


def hptq_synthetic_code():
    """(integers, lengths, codewords) in canonical order: sorted by (length, integer);
    each codeword is the previous plus 1, shifted left by the growth in length."""
    sym, ln = [], []
    for a, b, l in _HPTQ_CLASSES:
        vals = [0] if a == 0 else list(range(-b, -a + 1)) + list(range(a, b + 1))
        for v in vals:
            sym.append(v); ln.append(l)
    order = sorted(range(len(sym)), key=lambda k: (ln[k], sym[k]))
    sym = np.array([sym[k] for k in order], dtype=np.int64)
    ln = np.array([ln[k] for k in order], dtype=np.int64)
    codes = np.zeros(len(sym), dtype=np.int64)
    for k in range(1, len(sym)):
        codes[k] = (codes[k - 1] + 1) << (ln[k] - ln[k - 1])
    return sym, ln, codes


def hptq_stream(q: np.ndarray, sym, ln, codes):
    """Stream bytes (codewords most significant bit first, row by row) and row_bits [M+1]."""
    M, K = q.shape
    L = np.zeros(512, np.int64); C = np.zeros(512, np.int64)
    L[sym + 256] = ln; C[sym + 256] = codes
    lq = L[q.ravel() + 256]; cq = C[q.ravel() + 256]
    start = np.cumsum(lq) - lq
    row_bits = np.concatenate([[0], np.cumsum(lq.reshape(M, K).sum(axis=1))]).astype(np.int64)
    bits = np.zeros(int(row_bits[-1] + 7) // 8 * 8, dtype=np.uint8)
    for b in range(int(ln.max())):
        m = lq > b
        bits[start[m] + b] = ((cq[m] >> (lq[m] - 1 - b)) & 1).astype(np.uint8)
    return np.packbits(bits), row_bits


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def layer_shape(wl: Workload, layer: int = 0) -> tuple:
    """(M, K) of a layer; single-layer workloads have only layer 0."""
    if wl.layers:
        _, M, K = wl.layers[layer]
        return M, K
    if layer != 0:
        raise ValueError(f"{wl.name} has a single layer")
    return wl.M, wl.K


def outlier_count(wl: Workload, M: int, K: int) -> int:
    """Number of planted outliers: density * M * K rounded half-up."""
    return int(np.floor(wl.density * M * K + 0.5))


def _rng(wl: Workload, layer: int, stream: int, M: int, K: int) -> np.random.Generator:
    return np.random.default_rng([wl.wid, layer, stream, M, K])


def _top_n_linear(a: np.ndarray, n: int) -> np.ndarray:
    """Linear indices of the n largest entries of a (ties: lower index first), sorted."""
    order = np.argsort(-a.ravel(), kind="stable")[:n]
    return np.sort(order)


def _signed_uniform(rng: np.random.Generator, n: int) -> np.ndarray:
    """+-U(0.2, 2.5) with an independent, equiprobable sign."""
    mag = rng.uniform(0.2, 2.5, size=n)
    sign = np.where(rng.integers(0, 2, size=n) == 1, 1.0, -1.0)
    return sign * mag


def _row_skewed_positions(wl, rng, M, K, n):
    """2 full columns + heavy rows (5 % of rows) carrying 10x the density.

    The entries left after the two columns are shared out per row in
    proportion 10:1 (heavy:normal) by largest remainder (ties: lower row).
    Within a row the positions are uniform over the K-2 other columns.
    """
    full_cols = np.sort(rng.choice(K, size=min(2, K), replace=False))
    n_heavy = int(np.floor(0.05 * M + 0.5))
    heavy = np.zeros(M, dtype=bool)
    heavy[rng.choice(M, size=n_heavy, replace=False)] = True
    rest = max(0, n - len(full_cols) * M)
    w = np.where(heavy, 10.0, 1.0)
    share = rest * w / w.sum()
    counts = np.floor(share).astype(np.int64)
    left = rest - int(counts.sum())
    if left > 0:
        frac = share - counts
        order = np.argsort(-frac, kind="stable")[:left]
        counts[order] += 1
    other = np.setdiff1d(np.arange(K), full_cols)
    counts = np.minimum(counts, len(other))
    rows, cols = [], []
    for i in range(M):
        c = np.sort(np.concatenate([full_cols, rng.choice(other, size=counts[i], replace=False)]))
        rows.append(np.full(len(c), i, dtype=np.int64))
        cols.append(c)
    return np.concatenate(rows), np.concatenate(cols)


@lru_cache(maxsize=8)
def _make_weights_cached(name: str, layer: int, M: int, K: int):
    wl = WORKLOADS[name]
    n = outlier_count(wl, M, K)
    W = wl.sigma * _rng(wl, layer, 0, M, K).standard_normal((M, K))
    r_pos = _rng(wl, layer, 1, M, K)
    r_val = _rng(wl, layer, 2, M, K)
    if wl.law == "top_bulk":
        lin = _top_n_linear(np.abs(W), n)
        vals = _signed_uniform(r_val, len(lin))
    elif wl.law == "student_t_top":
        T = 0.1 * r_pos.standard_t(3, size=(M, K))
        lin = _top_n_linear(np.abs(T), n)
        vals = T.ravel()[lin]
    elif wl.law == "uniform_pos":
        lin = np.sort(r_pos.choice(M * K, size=n, replace=False))
        vals = _signed_uniform(r_val, len(lin))
    elif wl.law == "row_skewed":
        rows, cols = _row_skewed_positions(wl, r_pos, M, K, n)
        lin = rows * K + cols
        vals = _signed_uniform(r_val, len(lin))
    else:
        raise ValueError(wl.law)
    flat = W.ravel()
    flat[lin] = vals
    W16 = flat.reshape(M, K).astype(np.float16)
    planted = np.zeros(M * K, dtype=bool)
    planted[lin] = True
    planted = planted.reshape(M, K)
    # The planted entries are exactly the largest |w| of the FP16 matrix.
    a = np.abs(W16.astype(np.float64))
    if planted.any() and (~planted).any():
        assert a[planted].min() > a[~planted].max(), "planted outliers overlap the bulk"
    W16.setflags(write=False)
    planted.setflags(write=False)
    return W16, planted


def make_weights(wl: Workload | str, layer: int = 0, M: int | None = None, K: int | None = None):
    """FP16 weight matrix [M, K] with planted outliers, and the planted mask.

    Placement laws:
      top_bulk       the n largest |bulk| entries are replaced by +-U(0.2, 2.5)
      student_t_top  T = 0.1 * t(3) over the whole matrix; the n largest |T|
                     entries take the value T
      uniform_pos    n positions uniform without replacement, +-U(0.2, 2.5)
      row_skewed     see _row_skewed_positions, +-U(0.2, 2.5)
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    dM, dK = layer_shape(wl, layer)
    return _make_weights_cached(wl.name, layer, M or dM, K or dK)


def make_x(wl: Workload | str, B: int, K: int, layer: int = 0, M: int | None = None) -> np.ndarray:
    """Activations x, FP16 N(0, 1), shape [B, K].  Row 0 is the same for every B."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    dM, _ = layer_shape(wl, layer)
    rng = _rng(wl, layer, 3, M or dM, K)
    return rng.standard_normal((B, K)).astype(np.float16)


def make_format_inputs(wl: Workload | str, layer: int = 0, M: int | None = None, K: int | None = None):
    """Random arrays already in the storage format, for timing at full size.

    Codes are uniformly random bytes (every bit pattern of the per-row
    bitstream is a valid sequence of b-bit codes).  Uniform workloads get
    positive FP16 scales and integer-valued FP16 zero points in [0, 2^b - 1];
    BPDQ workloads get per-group coefficients C0 ~ -U(3, 4) sigma and
    C_t ~ U(0.5, 1.5) 2^(t-1) sigma;
    LUT workloads get one ascending FP16 table per row holding an exact 0.0
    and 2^b - 1 Gaussian draws.  Outlier positions follow the workload's
    placement law (value-ranked laws are drawn uniformly, which gives the same
    count and the same per-row distribution for an i.i.d. bulk); outlier
    values are FP16 +-U(0.2, 2.5).  Returned positions are row-major sorted.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    dM, dK = layer_shape(wl, layer)
    M = M or dM
    K = K or dK
    rng = _rng(wl, layer, 4, M, K)
    out = {"M": M, "K": K, "bits": wl.bits, "fmt": wl.fmt, "group": wl.group}
    out["codes_packed"] = rng.integers(0, 256, size=(M, K * wl.bits // 8), dtype=np.uint8)
    levels = 1 << wl.bits
    if wl.fmt == "uniform":
        G = K // wl.group
        out["scales"] = (rng.uniform(0.5, 1.5, size=(M, G)) * 4 * wl.sigma / (levels - 1)).astype(np.float16)
        out["zeros"] = rng.integers(0, levels, size=(M, G)).astype(np.float16)
    elif wl.fmt == "hptq":
        # integers rint(N(0, 1.5)) (|q| <= 255), steps ~ U(0.5, 1.5) * sigma / 1.5 per row and group of 128,
        # and the outliers as large integers on the same grid
        G = K // wl.group
        q = np.clip(np.rint(rng.standard_normal((M, K)) * 1.5), -255, 255).astype(np.int64)
        out["scales"] = (rng.uniform(0.5, 1.5, size=(M, G)) * wl.sigma / 1.5).astype(np.float16)
        n = outlier_count(wl, M, K)
        lin = np.sort(_rng(wl, layer, 1, M, K).choice(M * K, size=n, replace=False))
        mag = _rng(wl, layer, 2, M, K).integers(32, 256, size=n)
        q.ravel()[lin] = np.where(np.arange(n) % 2 == 0, mag, -mag)
        sym, ln, codes = hptq_synthetic_code()
        out["stream"], out["row_bits"] = hptq_stream(q, sym, ln, codes)
        del out["codes_packed"]
        out["huff_sym"] = sym.astype(np.int16)
        out["huff_len"] = ln.astype(np.uint8)
        out["q"] = q
        out["rows"] = np.zeros(0, np.int64); out["cols"] = np.zeros(0, np.int64)
        out["values"] = np.zeros(0, np.float16)
        return out
    elif wl.fmt == "bpdq":
        G = K // wl.group
        c = np.empty((M, G, wl.bits + 1))
        c[:, :, 0] = -rng.uniform(3.0, 4.0, size=(M, G)) * wl.sigma
        for t in range(1, wl.bits + 1):
            c[:, :, t] = rng.uniform(0.5, 1.5, size=(M, G)) * (1 << (t - 1)) * wl.sigma
        out["coefs"] = c.astype(np.float16)
    else:
        draws = rng.standard_normal((M, levels - 1)) * 2 * wl.sigma
        lut = np.concatenate([draws, np.zeros((M, 1))], axis=1).astype(np.float16)
        out["lut"] = np.sort(lut, axis=1)
    n = outlier_count(wl, M, K)
    r_pos = _rng(wl, layer, 1, M, K)
    if wl.law == "row_skewed":
        rows, cols = _row_skewed_positions(wl, r_pos, M, K, n)
    else:
        lin = np.sort(r_pos.choice(M * K, size=n, replace=False))
        rows, cols = lin // K, lin % K
    out["rows"] = rows.astype(np.int64)
    out["cols"] = cols.astype(np.int64)
    out["values"] = _signed_uniform(_rng(wl, layer, 2, M, K), len(rows)).astype(np.float16)
    return out
