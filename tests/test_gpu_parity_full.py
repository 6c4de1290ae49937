"""GPU parity at the workloads' full sizes: every output row and every code.

Two kinds of input:

* the arrays bench.py times (random arrays in the storage format with each
  workload's shapes, tables, statistics and outlier placement law), run in
  the same launch configuration, at the batch sizes the workloads name;
* the oracle's own encodings of the workloads' weight laws: the 4096x4096
  uniform-3 attention projection, the 11008x4096 LUT-3 MLP, a full-width
  2048x8192 slice of the 70B LUT-4 MLP (row-skewed outliers and two full
  columns), and one 7B-block layer of each shape at batch 16 (and 1).

Every output is checked against |y_gpu - y| <= 1e-4 A + 1e-6 with the
oracle run in row chunks; every code of qgemv_debug_unpack must equal the
canonical one.  Outputs are framed by canary words and must be written
exactly once and deterministically.
"""

import numpy as np
import pytest

from dense_sparse_bit_amd import qgemv
from encode_pool import encode_workload
from gpu_checks import check_all, run_framed, say, unpack_framed
from synth import make_format_inputs, make_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    return t


def format_case(name, layer=0):
    f = make_format_inputs(name, layer)
    counts = np.bincount(f["rows"], minlength=f["M"])
    f["row_ptr"] = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    f["col_idx"] = f["cols"].astype(np.int32)
    f["values"] = np.asarray(f["values"], np.float16)
    return f


FORMAT_CASES = [
    ("tiny_u4", 0, (1,)),
    ("attn7b_u3", 0, (1,)),
    ("mlp7b_lut3", 0, (1,)),
    ("mlp70b_lut4", 0, (1, 8)),
    ("block7b_u3", 0, (16, 1)),
    ("block7b_u3", 4, (16, 1)),
    ("block7b_u3", 6, (16, 1)),
    ("mlp7b_bpdq3", 0, (1, 8)),
]


@pytest.mark.parametrize("name,layer,batches", FORMAT_CASES)
def test_bench_inputs_every_row(torch, name, layer, batches):
    f = format_case(name, layer)
    M, K = f["M"], f["K"]
    say(f"[gpu] full-size bench input {name} layer={layer} M={M} K={K} nnz={f['row_ptr'][-1]} B={batches}")
    plan = qgemv.QGemv(f)
    codes = unpack_framed(torch, plan)
    runs = []
    for B in batches:
        x16 = make_x(name, B, K, layer, M)
        y = run_framed(torch, plan, x16)
        assert np.array_equal(y, run_framed(torch, plan, x16)), f"B={B}: not bitwise deterministic"
        runs.append((y, x16))
    worst = check_all(codes, runs, f)
    say(f"[gpu]   worst |dy|/tol = {worst:.3e}")
    plan.close()


ORACLE_CASES = [
    ("attn7b_u3", 0, None, None, (1,)),
    ("mlp7b_lut3", 0, None, None, (1,)),
    ("mlp70b_lut4", 0, 2048, 8192, (1, 8)),
    ("block7b_u3", 0, None, None, (16, 1)),
    ("block7b_u3", 4, None, None, (16, 1)),
    ("block7b_u3", 6, None, None, (16, 1)),
]


@pytest.mark.parametrize("name,layer,M,K,batches", ORACLE_CASES)
def test_oracle_encoded_every_row(torch, name, layer, M, K, batches):
    enc, xall = encode_workload(name, layer, M, K)
    M_, K_ = enc["M"], enc["K"]
    say(f"[gpu] full-size oracle encoding {name} layer={layer} M={M_} K={K_} nnz={enc['row_ptr'][-1]} B={batches}")
    plan = qgemv.QGemv(enc)
    codes = unpack_framed(torch, plan)
    runs = []
    for B in batches:
        x16 = np.ascontiguousarray(xall[:B]) if B <= xall.shape[0] else make_x(name, B, K_, layer, M_)
        y = run_framed(torch, plan, x16)
        assert np.array_equal(y, run_framed(torch, plan, x16)), f"B={B}: not bitwise deterministic"
        runs.append((y, x16))
    worst = check_all(codes, runs, enc)
    say(f"[gpu]   worst |dy|/tol = {worst:.3e}")
    plan.close()


# Layers that read the same x, run as one product over their stacked rows
# (bench.py --fuse): each part of y is checked against its own layer's oracle.
STACKED_CASES = [
    ("block7b_u3", (0, 1, 2), (16, 1)),
    ("block7b_u3", (4, 5), (16, 1)),
]


@pytest.mark.parametrize("name,layers,batches", STACKED_CASES)
def test_stacked_layers_every_row(torch, name, layers, batches):
    import bench
    parts = [format_case(name, i) for i in layers]
    f = bench.stack_rows(parts)
    M, K = f["M"], f["K"]
    say(f"[gpu] stacked bench inputs {name} layers={layers} M={M} K={K} nnz={f['row_ptr'][-1]} B={batches}")
    plan = qgemv.QGemv(f)
    codes = unpack_framed(torch, plan)
    runs = []
    for B in batches:
        x16 = make_x(name, B, K, layers[0], parts[0]["M"])
        y = run_framed(torch, plan, x16)
        assert np.array_equal(y, run_framed(torch, plan, x16)), f"B={B}: not bitwise deterministic"
        runs.append((y, x16))
    worst, r0 = 0.0, 0
    for p in parts:
        rows = slice(r0, r0 + p["M"])
        w = check_all(codes[rows], [(y[:, rows], x16) for y, x16 in runs], p)
        worst = max(worst, w)
        r0 += p["M"]
    say(f"[gpu]   worst |dy|/tol = {worst:.3e}")
    plan.close()
