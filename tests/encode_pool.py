"""Oracle encodings of whole workload matrices, row chunks in worker processes.

Test infrastructure (not collected).  The oracle's only step that looks
across rows is the magnitude outlier pick; everything after it (the dense
quantization and the CSR residual) works row by row.  The generator plants
outliers strictly above the bulk in magnitude, so the pick over any set of
rows is the planted set of those rows.  Encoding row chunks on their own, each
with its own planted count, therefore gives exactly the whole matrix's
encoding (tests/test_encode_pool.py checks that equality on the CPU).
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from oracle import encode
from synth import WORKLOADS, make_weights, make_x, outlier_count


def workers() -> int:
    """Host threads of this process, at most 16 (the GPU machine's share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _encode_chunk(args):
    W, bits, fmt, n, group, sens = args
    return encode.encode(W, bits, fmt, n, group, sens=sens)


def _concat(parts, M, K, bits, fmt, group):
    out = {"M": M, "K": K, "bits": bits, "fmt": fmt, "group": parts[0]["group"]}
    for key in ("codes", "codes_packed", "mask", "scales", "zeros", "lut", "coefs"):
        if key in parts[0]:
            out[key] = np.concatenate([p[key] for p in parts], axis=0)
    nnz = np.cumsum([0] + [int(p["row_ptr"][-1]) for p in parts])
    out["row_ptr"] = np.concatenate([[0]] + [p["row_ptr"][1:] + nnz[k] for k, p in enumerate(parts)]).astype(np.int32)
    out["col_idx"] = np.concatenate([p["col_idx"] for p in parts]).astype(np.int32)
    out["values"] = np.concatenate([p["values"] for p in parts]).astype(np.float16)
    return out


def encode_rows(W16, planted, bits, fmt, group, sens, chunk=256, nproc=None):
    """encode.encode of the whole matrix, computed in row chunks (see the module docstring)."""
    M, K = W16.shape
    bounds = [(r, min(M, r + chunk)) for r in range(0, M, chunk)]
    jobs = [(np.ascontiguousarray(W16[a:b]), bits, fmt, int(planted[a:b].sum()), group, sens) for a, b in bounds]
    nproc = nproc or workers()
    if nproc == 1 or len(jobs) == 1:
        parts = [_encode_chunk(j) for j in jobs]
    else:
        with mp.get_context("spawn").Pool(nproc) as pool:
            parts = pool.map(_encode_chunk, jobs, chunksize=1)
    return _concat(parts, M, K, bits, fmt, group)


def encode_workload(name, layer=0, M=None, K=None, batch=None, chunk=256, nproc=None):
    """(encoding, x [B, K]) of a workload's weight law at the given shape; the
    LUT sensitivities are x[0]^2 (x of the workload's largest batch, row 0)."""
    wl = WORKLOADS[name]
    W, planted = make_weights(wl, layer, M, K)
    M_, K_ = W.shape
    assert int(planted.sum()) == outlier_count(wl, M_, K_)
    x = make_x(wl, batch or max(wl.batches), K_, layer, M_)
    sens = x[0].astype(np.float64) ** 2
    enc = encode_rows(W, planted, wl.bits, wl.fmt, wl.group or 16, sens, chunk=chunk, nproc=nproc)
    return enc, x
