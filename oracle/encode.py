"""Oracle encoder: W (FP16) -> dense codes + statistics/LUT + CSR outliers, in fp64.

Test infrastructure only (see the package docstring).

Step order follows the pages:
  1. outlier pick                      [SpQR] "Qu'est-ce qu'un poids outlier ?" (magnitude)
                                       [SqLLM] "Sélection des outliers" (sensitivity-weighted error)
                                       [Babai/GPTQ] SSQR (overflows of shrunk uniform grids)
  2. dense part with holes, quantized  [SpQR] "La solution SpQR : décomposition sparse + dense",
                                              "Quantification d'un modèle" (wbits, groupsize 16)
                                       [SqLLM] "Non-uniform quantization via Lloyd-Max optimisé"
                                       [BPDQ] "Formulation de la Grille Variable", "Cadre d'Optimisation"
  3. sparse residual in CSR            [SpQR] "Le format de stockage sparse"
                                       [SqLLM] "2. Dense-and-Sparse decomposition" (W = W_dense + W_sparse)

Readings taken where the pages are silent are listed next to each function.
"""

from __future__ import annotations

import numpy as np

from .pack import pack_bitstream

FP16_MIN_SUBNORMAL = 2.0 ** -24


def f16(a):
    """Round to IEEE binary16 (round-to-nearest-even) and return it as fp64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# 1. Outlier pick
# --------------------------------------------------------------------------
def pick_outliers(W16: np.ndarray, n: int) -> np.ndarray:
    """Boolean mask of the n weights of largest |w|.

    [SpQR] "Qu'est-ce qu'un poids outlier ?": outliers are the few weights of
    abnormally large magnitude in an otherwise Gaussian matrix.  Reading: the
    count n comes from the workload's density; ties go to the lower row-major
    index.
    """
    a = np.abs(W16.astype(np.float64)).ravel()
    mask = np.zeros(a.size, dtype=bool)
    if n > 0:
        order = np.argsort(-a, kind="stable")[:n]
        mask[order] = True
    return mask.reshape(W16.shape)


def first_pass_error(W16: np.ndarray, sens: np.ndarray, bits: int) -> np.ndarray:
    """Per-weight sensitivity-weighted error s_j (w_ij - q(w_ij))^2 of a first-pass LUT.

    [SqLLM] "Sélection des outliers": the criterion is the quantization error
    weighted by the weight's sensitivity.  Reading: q is the row's LUT fitted
    by lloyd_row over all of the row's weights (no holes yet), rounded to FP16,
    each weight taking its nearest entry (ties: lower entry).
    """
    M, K = W16.shape
    W = W16.astype(np.float64)
    s = np.asarray(sens, dtype=np.float64)
    err = np.zeros((M, K))
    for i in range(M):
        cent, _ = lloyd_row(W[i], s, 1 << bits)
        tab = np.sort(cent.astype(np.float16), kind="stable").astype(np.float64)
        err[i] = s * (W[i] - tab[nearest(W[i], tab)]) ** 2
    return err


def pick_outliers_sensitivity(W16: np.ndarray, sens: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Boolean mask of the n weights of largest sensitivity-weighted first-pass error.

    [SqLLM] "Sélection des outliers": a weight goes to the sparse part when
    s_i (w_i - q(w_i))^2 exceeds a threshold, so a moderate weight of very
    high sensitivity can be extracted too, not only large ones.  Reading: the
    threshold is the one that extracts exactly n weights (the workload's
    density), i.e. the n largest errors, ties to the lower row-major index.
    The LUT is then fitted again without these weights (quant_lut with them
    as holes), as the dense part is quantized after the decomposition.
    """
    e = first_pass_error(W16, sens, bits).ravel()
    mask = np.zeros(e.size, dtype=bool)
    if n > 0:
        order = np.argsort(-e, kind="stable")[:n]
        mask[order] = True
    return mask.reshape(W16.shape)


# --------------------------------------------------------------------------
# 2a. Uniform asymmetric group quantization
# --------------------------------------------------------------------------
def quant_uniform(W16: np.ndarray, hole: np.ndarray, bits: int, group: int):
    """Asymmetric min-max round-to-nearest per group of `group` weights along K.

    [SpQR] "Quantification d'un modèle": 3-4 bit dense part, groupsize 16.
    Each (row, group) keeps an FP16 scale and an FP16 zero point.

    Per group, with L = 2^bits - 1 and D the group's non-outlier values:
      lo = min(0, min D), hi = max(0, max D)   (lo = hi = 0 if D is empty)
      if hi == lo: scale = 1, z = 0
      else: scale = fp16((hi - lo) / L)  (2^-24 if that rounds to 0)
            z = clamp(rint(-lo / scale), 0, L)      -- an exact integer
      q = clamp(rint(w / scale) + z, 0, L) for non-outliers
      q = z at outlier positions (the "holes", which then decode to exactly 0)
    Decode: d = scale * (q - z).

    Readings: the range includes 0 and the zero point is an integer so that a
    hole decodes to exactly 0 (then W_dense + W_sparse reproduces W exactly);
    rint rounds half to even.

    Returns (codes uint8 [M, K], scales fp16 [M, K/group], zeros fp16 [M, K/group]).
    """
    M, K = W16.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    L = (1 << bits) - 1
    w = W16.astype(np.float64).reshape(M, G, group)
    h = hole.reshape(M, G, group)
    lo = np.minimum(0.0, np.min(np.where(h, np.inf, w), axis=2))
    hi = np.maximum(0.0, np.max(np.where(h, -np.inf, w), axis=2))
    flat = hi == lo
    scale = f16((hi - lo) / L)
    scale = np.where(scale == 0.0, FP16_MIN_SUBNORMAL, scale)
    scale = np.where(flat, 1.0, scale)
    if not np.all(np.isfinite(scale)):
        raise ValueError("group range overflows FP16")
    z = np.where(flat, 0.0, np.clip(np.rint(-lo / scale), 0, L))
    q = np.clip(np.rint(w / scale[..., None]) + z[..., None], 0, L)
    q = np.where(h, z[..., None], q)
    return (q.reshape(M, K).astype(np.uint8),
            scale.astype(np.float16),
            z.astype(np.float16))


# --------------------------------------------------------------------------
# 2a'. SSQR: shrunk uniform grids, overflowing weights to the sparse part
# --------------------------------------------------------------------------
def quant_uniform_scaled(W16: np.ndarray, bits: int, group: int, alpha: float):
    """Uniform group quantization on a grid shrunk by alpha; overflows become outliers.

    [Babai/GPTQ] "3. Applications Pratiques et Algorithmes", SSQR: a scheme
    that tolerates overflow -- weights that do not fit the integer grid are
    kept in full precision in the sparse part instead of being clipped.

    Per group, with L = 2^bits - 1, over all of the group's values (0 included):
      lo = min(0, min w), hi = max(0, max w)
      if hi == lo: scale = 1, z = 0 (nothing overflows)
      else: scale = fp16(alpha * (hi - lo) / L)  (2^-24 if that rounds to 0)
            z = clamp(rint(-alpha * lo / scale), 0, L)
      t = rint(w / scale) + z; a weight overflows when t < 0 or t > L.
      q = t for the others; q = z at overflows (holes, decoding to exactly 0).
    Readings: one factor alpha for the whole matrix scales every group's
    min-max grid about zero; the zero point is the integer nearest to the
    shrunk lower end.

    Returns (codes uint8 [M, K], scales fp16 [M, K/group], zeros fp16 [M, K/group],
    overflow mask bool [M, K]).
    """
    M, K = W16.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    L = (1 << bits) - 1
    w = W16.astype(np.float64).reshape(M, G, group)
    lo = np.minimum(0.0, w.min(axis=2))
    hi = np.maximum(0.0, w.max(axis=2))
    flat = hi == lo
    scale = f16(np.where(flat, 1.0, alpha * (hi - lo) / L))
    scale = np.where(scale == 0.0, FP16_MIN_SUBNORMAL, scale)
    z = np.where(flat, 0.0, np.clip(np.rint(-alpha * lo / scale), 0, L))
    t = np.rint(w / scale[:, :, None]) + z[:, :, None]
    over = (t < 0) | (t > L)
    q = np.where(over, z[:, :, None], t)
    return (q.reshape(M, K).astype(np.uint8), scale.astype(np.float16), z.astype(np.float16),
            over.reshape(M, K))


def ssqr_alpha(W16: np.ndarray, bits: int, group: int, n: int, iters: int = 40) -> float:
    """Binary search for the grid factor that meets the outlier budget.

    [Babai/GPTQ] "3. Applications Pratiques et Algorithmes", SSQR: a binary
    search adjusts the scales to reach a target outlier density.  Reading:
    the result is the smallest alpha in (0, 1] (to `iters` halvings) whose
    overflow count is at most n, i.e. the finest grids within the budget; the
    count falls as alpha grows.  Returns 1.0 if even alpha = 1 overflows more
    than n times.
    """
    count = lambda a: int(quant_uniform_scaled(W16, bits, group, a)[3].sum())
    if count(1.0) > n:
        return 1.0
    lo_a, hi_a = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo_a + hi_a)
        if count(mid) <= n:
            hi_a = mid
        else:
            lo_a = mid
    return hi_a


# --------------------------------------------------------------------------
# 2c. BPDQ: bit planes on a variable grid
# --------------------------------------------------------------------------
def bpdq_levels(c: np.ndarray, k: int) -> np.ndarray:
    """The 2^k values of one group's grid: level(q) = C0 + sum_i C_i * bit_(i-1)(q).

    [BPDQ] "1. Formulation de la Grille Variable": W^ = REP(C0) + sum_i REP(C_i) (.) B_i
    with B_i in {0, 1}.  Reading: plane B_i of a weight is bit i-1 of its
    k-bit code (plane 1 the least significant).
    """
    q = np.arange(1 << k)
    lv = np.full(q.size, float(c[0]))
    for i in range(1, k + 1):
        lv = lv + float(c[i]) * ((q >> (i - 1)) & 1)
    return lv


def bpd_init(w: np.ndarray, k: int) -> np.ndarray:
    """Initial codes: the k most significant bit planes of the weights.

    [BPDQ] "2. Cadre d'Optimisation", initialisation: the planes come from the
    bit-plane decomposition of the weights, keeping the k most significant.
    Reading: a group's weights are mapped onto [0, 1] by its min and max; the
    code is the fraction's binary expansion cut to k bits,
    q = min(floor(2^k u), 2^k - 1) (all 0 if the group is constant).
    """
    lo, hi = float(w.min()), float(w.max())
    if hi == lo:
        return np.zeros(w.size, dtype=np.int64)
    u = (w - lo) / (hi - lo)
    return np.minimum(np.floor(u * (1 << k)), (1 << k) - 1).astype(np.int64)


def bpdq_fit(w: np.ndarray, q: np.ndarray, k: int) -> np.ndarray:
    """Coefficients (C0 .. Ck) minimising sum (w - level(q))^2, in fp64.

    [BPDQ] "2. Cadre d'Optimisation": scalar coefficients by an analytic
    least-squares fit.  Reading: no calibration data here, so the Hessian
    metric is the identity and the fit is ordinary least squares on the design
    [1, B_1 .. B_k]; numpy's lstsq gives the minimum-norm solution when a plane
    is constant over the group.
    """
    A = np.stack([np.ones(w.size)] + [((q >> (i - 1)) & 1).astype(np.float64) for i in range(1, k + 1)], axis=1)
    return np.linalg.lstsq(A, w, rcond=None)[0]


def bpdq_assign(w: np.ndarray, c: np.ndarray, k: int) -> np.ndarray:
    """Codes by exact enumeration of the 2^k bit patterns (ties: lower code).

    [BPDQ] "2. Cadre d'Optimisation", refinement step 1: for fixed
    coefficients the bit planes are updated by exact enumeration.  Reading:
    with the identity metric every weight is independent, so each takes the
    pattern whose level is nearest.
    """
    return nearest(w, bpdq_levels(c, k)).astype(np.int64)


def bpdq_group(w: np.ndarray, k: int, max_iter: int = 20, history: list | None = None):
    """One group: BPD initialisation, then alternate refits and bit updates.

    [BPDQ] "2. Cadre d'Optimisation": initialise the planes by BPD, fit the
    coefficients, then alternate (1) bit updates by enumeration and (2)
    least-squares refits.  Readings: stop when the codes no longer change or
    after max_iter rounds; the coefficients are then rounded to FP16 (the
    stored format) and the codes chosen once more against the rounded values.
    No delta correction: with the identity metric no error is propagated to
    other columns.
    Returns (codes int64, FP16 coefficients as fp64 [k+1]).
    If `history` is a list, the objective after every refit is appended.
    """
    if w.size == 0:
        return np.zeros(0, dtype=np.int64), np.zeros(k + 1)
    q = bpd_init(w, k)
    for _ in range(max_iter):
        c = bpdq_fit(w, q, k)
        if history is not None:
            history.append(float(np.sum((w - bpdq_levels(c, k)[q]) ** 2)))
        q2 = bpdq_assign(w, c, k)
        if np.array_equal(q2, q):
            break
        q = q2
    c16 = f16(bpdq_fit(w, q, k))
    return bpdq_assign(w, c16, k), c16


def quant_bpdq(W16: np.ndarray, hole: np.ndarray, bits: int, group: int):
    """BPDQ dense part: per (row, group of `group` columns) FP16 coefficients and k-bit codes.

    The fit uses the group's non-outlier weights.  At an outlier position the
    code is the one whose level is nearest 0 (ties: lower code); the CSR then
    holds the residual fp16(w - level) (build_csr), so W_dense + W_sparse
    reproduces the outlier to FP16 rounding of the residual.

    Returns (codes uint8 [M, K], coefs fp16 [M, K/group, bits+1]).
    """
    M, K = W16.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    W = W16.astype(np.float64)
    codes = np.zeros((M, K), dtype=np.uint8)
    coefs = np.zeros((M, G, bits + 1), dtype=np.float16)
    for i in range(M):
        for g in range(G):
            sl = slice(g * group, (g + 1) * group)
            w, h = W[i, sl], hole[i, sl]
            q = np.zeros(group, dtype=np.int64)
            qk, c = bpdq_group(w[~h], bits)
            q[~h] = qk
            q[h] = int(np.argmin(np.abs(bpdq_levels(c, bits))))
            codes[i, sl] = q
            coefs[i, g] = c.astype(np.float16)
    return codes, coefs


# --------------------------------------------------------------------------
# 2b. Sensitivity-weighted Lloyd-Max LUT (non-uniform)
# --------------------------------------------------------------------------
def weighted_quantile(w: np.ndarray, s: np.ndarray, qs) -> np.ndarray:
    """Lower inverse CDF of the s-weighted empirical distribution of w.

    For each level q: the smallest w (in sorted order) whose cumulative weight
    fraction reaches q.
    """
    order = np.argsort(w, kind="stable")
    ws, ss = w[order], s[order]
    cw = np.cumsum(ss) / ss.sum()
    idx = np.searchsorted(cw, np.asarray(qs, dtype=np.float64), side="left")
    return ws[np.minimum(idx, len(ws) - 1)]


def weighted_sse(w, s, cent, assign):
    """Objective of [SqLLM] "Non-uniform quantization via Lloyd-Max optimisé": sum_i s_i (w_i - q(w_i))^2."""
    return float(np.sum(s * (w - cent[assign]) ** 2))


def nearest(w: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid by |w - c|; ties go to the lower index."""
    return np.argmin(np.abs(w[:, None] - cent[None, :]), axis=1)


def lloyd_row(w: np.ndarray, s: np.ndarray, C: int, max_iter: int = 100, history: list | None = None):
    """Weighted Lloyd-Max on one row, with one centroid pinned at +0.0.

    [SqLLM] "Non-uniform quantization via Lloyd-Max optimisé": minimise
    sum_i s_i (w_i - q(w_i))^2 by (1) initialising the bins from statistics,
    (2) assigning every weight to its nearest bin, (3) moving each bin centre
    to the s-weighted mean of its weights, (4) repeating until convergence.

    Readings:
      * one of the C centroids is pinned at +0.0 and never moves (the hole
        code must decode to exactly 0);
      * initial free centroids: weighted quantiles at levels (k + 1/2)/(C - 1),
        k = 0..C-2 (unweighted if every sensitivity is 0);
      * assignment to the nearest centroid, ties to the lower one (a positive
        per-weight factor s_i does not change a 1-D nearest assignment);
      * a free centroid with zero total weight keeps its value;
      * convergence = no assignment changed; at most `max_iter` iterations.

    Returns (centroids sorted ascending as fp64, index of the pinned zero).
    If `history` is a list, the objective after every centroid update is appended.
    """
    if len(w) == 0:
        return np.zeros(C), 0
    levels = (np.arange(C - 1) + 0.5) / (C - 1)
    sw = s if s.sum() > 0 else np.ones_like(s)
    cent = np.concatenate([[0.0], weighted_quantile(w, sw, levels)])
    pinned = np.zeros(C, dtype=bool)
    pinned[0] = True
    prev = None
    for _ in range(max_iter):
        order = np.argsort(cent, kind="stable")
        cent, pinned = cent[order], pinned[order]
        a = nearest(w, cent)
        if prev is not None and np.array_equal(a, prev):
            break
        for c in range(C):
            if pinned[c]:
                continue
            sel = a == c
            tot = s[sel].sum()
            if tot > 0:
                cent[c] = np.sum(s[sel] * w[sel]) / tot
        if history is not None:
            history.append(weighted_sse(w, s, cent, a))
        prev = a
    order = np.argsort(cent, kind="stable")
    cent, pinned = cent[order], pinned[order]
    return cent, int(np.flatnonzero(pinned)[0])


def quant_lut(W16: np.ndarray, hole: np.ndarray, sens: np.ndarray, bits: int):
    """Per-output-row non-uniform LUT of 2^bits FP16 entries, and the codes.

    Sensitivity s_j is supplied per input column (the x^2 proxy: s_j = x_j^2).
    For row i the data are its non-outlier weights with their s_j.
      LUT_i = fp16(lloyd_row(...)) ascending
      q_ij  = argmin_c |w_ij - LUT_i[c]|  (ties: lower c) for non-outliers
      q_ij  = smallest c with LUT_i[c] == 0 at outlier positions (holes)
    Decode: d = LUT_i[q].

    Returns (codes uint8 [M, K], lut fp16 [M, 2^bits]).
    """
    M, K = W16.shape
    C = 1 << bits
    W = W16.astype(np.float64)
    codes = np.zeros((M, K), dtype=np.uint8)
    lut = np.zeros((M, C), dtype=np.float16)
    for i in range(M):
        keep = ~hole[i]
        cent, _ = lloyd_row(W[i, keep], sens[keep], C)
        tab16 = np.sort(cent.astype(np.float16), kind="stable")
        tab = tab16.astype(np.float64)
        q = nearest(W[i], tab).astype(np.uint8)
        zero_code = int(np.flatnonzero(tab == 0.0)[0])
        q[hole[i]] = zero_code
        codes[i] = q
        lut[i] = tab16
    return codes, lut


# --------------------------------------------------------------------------
# 3. Sparse residual in CSR
# --------------------------------------------------------------------------
def build_csr(W16: np.ndarray, hole: np.ndarray, D: np.ndarray):
    """CSR of the residual r = fp16(w - d) at the outlier positions.

    [SpQR] "Le format de stockage sparse": values (FP16), col_idx, row_ptr.
    Entries in row-major order, columns ascending inside a row; int32 indices;
    row_ptr[0] = 0 and row_ptr[i+1] = row_ptr[i] + (outliers in row i).
    Because holes decode to exactly 0, r equals the original FP16 weight.
    """
    M, K = W16.shape
    rows, cols = np.nonzero(hole)            # row-major, ascending columns
    w = W16.astype(np.float64)[rows, cols]
    d = D[rows, cols]
    values = (w - d).astype(np.float16)
    counts = np.bincount(rows, minlength=M)
    row_ptr = np.zeros(M + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr, cols.astype(np.int32), values


# --------------------------------------------------------------------------
# Whole encoder
# --------------------------------------------------------------------------
def encode(W16: np.ndarray, bits: int, fmt: str, n_outliers: int, group: int = 16,
           sens: np.ndarray | None = None, pick: str = "magnitude") -> dict:
    """Encode an FP16 matrix into the canonical dense-and-sparse format.

    pick: "magnitude" (pick_outliers), "sensitivity" (pick_outliers_sensitivity,
    LUT format only: it needs the sensitivities and a first-pass LUT) or "ssqr"
    (uniform format only: the overflows of the grids ssqr_alpha finds for a
    budget of n_outliers, which are then the outliers and the grids the dense part).

    Returns a dict with the fields of the canonical format:
      M, K, bits, fmt, group, codes (uint8 [M,K], unpacked), codes_packed
      (uint8 [M, K*bits/8]), scales/zeros (uniform) or lut (LUT), row_ptr,
      col_idx, values, and the outlier mask.
    """
    from .gemv import decode
    M, K = W16.shape
    ssqr = None
    if pick == "magnitude":
        hole = pick_outliers(W16, n_outliers)
    elif pick == "ssqr":
        if fmt != "uniform":
            raise ValueError("the SSQR pick needs the uniform format")
        alpha = ssqr_alpha(W16, bits, group, n_outliers)
        ssqr = quant_uniform_scaled(W16, bits, group, alpha)
        hole = ssqr[3]
    elif pick == "sensitivity":
        if fmt != "lut" or sens is None:
            raise ValueError("the sensitivity pick needs the LUT format and a sensitivity vector")
        hole = pick_outliers_sensitivity(W16, np.asarray(sens, dtype=np.float64), bits, n_outliers)
    else:
        raise ValueError(pick)
    out = {"M": M, "K": K, "bits": bits, "fmt": fmt, "group": group if fmt == "uniform" else 0,
           "mask": hole}
    if fmt == "uniform":
        if ssqr is not None:
            codes, scales, zeros = ssqr[:3]
            out["alpha"] = alpha
        else:
            codes, scales, zeros = quant_uniform(W16, hole, bits, group)
        out.update(scales=scales, zeros=zeros)
    elif fmt == "lut":
        if sens is None:
            raise ValueError("LUT quantization needs a sensitivity vector")
        codes, lut = quant_lut(W16, hole, np.asarray(sens, dtype=np.float64), bits)
        out.update(lut=lut)
    elif fmt == "bpdq":
        codes, coefs = quant_bpdq(W16, hole, bits, group)
        out.update(coefs=coefs, group=group)
    else:
        raise ValueError(fmt)
    out["codes"] = codes
    out["codes_packed"] = pack_bitstream(codes, bits)
    D = decode(out)
    out["row_ptr"], out["col_idx"], out["values"] = build_csr(W16, hole, D)
    return out
