"""qgemv_run_noalloc (no device allocation; the library's static scratch)
against qgemv_run (the plan's workspace), through the C ABI.

Two calls in a row on one device, the second with a smaller input, both
bitwise equal to qgemv_run's output and within the oracle's tolerance; a
batch-1 call; a shape that needs more than the static scratch is refused.
"""

import ctypes

import numpy as np
import pytest

from dense_sparse_bit_amd import qgemv
from gpu_checks import run_framed, say
from oracle import encode, gemv
from synth import WORKLOADS, make_weights, make_x, outlier_count

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    return t


def _noalloc_framed(torch, plan, x16):
    """qgemv_run_noalloc into a NaN-filled y framed by canaries (as run_framed)."""
    from gpu_checks import CANARY, PAD
    x = torch.from_numpy(np.ascontiguousarray(x16)).cuda()
    B = x16.shape[0]
    buf = torch.empty(2 * PAD + B * plan.M, dtype=torch.float32, device="cuda")
    buf.view(torch.int32).fill_(int(CANARY))
    y = buf[PAD:PAD + B * plan.M].view(B, plan.M)
    y.fill_(float("nan"))
    s = torch.cuda.current_stream().cuda_stream
    st = qgemv.lib().qgemv_run_noalloc(plan._h, x.data_ptr(), y.data_ptr(), B, s)
    assert st == 0, f"qgemv_run_noalloc: {st}"
    torch.cuda.synchronize()
    pads = buf.view(torch.int32).cpu().numpy()
    assert np.all(pads[:PAD] == CANARY) and np.all(pads[-PAD:] == CANARY), "write outside y"
    out = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out)), "output not fully written"
    return out


def _case(M, K, B):
    wl = WORKLOADS["block7b_u3"]
    W, _ = make_weights(wl, 0, M, K)
    enc = encode.encode(W, 3, "uniform", outlier_count(wl, M, K), 16)
    return enc, make_x(wl, B, K, 0, M)


def test_noalloc_matches_run_twice_then_smaller(torch):
    """Larger input first, then a smaller one: the scratch keeps the first
    call's contents, which must not leak into the second."""
    for M, K, B in ((1000, 2048, 16), (300, 1024, 8), (1000, 2048, 16)):
        enc, x16 = _case(M, K, B)
        say(f"[gpu] no-alloc uniform-3 M={M} K={K} B={B}")
        plan = qgemv.QGemv(enc)
        y_na = _noalloc_framed(torch, plan, x16)
        y_run = run_framed(torch, plan, x16)
        assert np.array_equal(y_na, y_run), "qgemv_run_noalloc differs from qgemv_run"
        y_ref, A = gemv.gemv(enc, x16)
        ok, worst = gemv.within_tolerance(y_na, y_ref, A)
        assert ok, f"tolerance exceeded: worst {worst:.3f}"
        # batch 1 needs no scratch: the same kernels as qgemv_run
        y1 = _noalloc_framed(torch, plan, x16[:1])
        assert np.array_equal(y1, run_framed(torch, plan, x16[:1]))
        plan.close()


def test_noalloc_refuses_shapes_beyond_the_scratch(torch):
    """66000 x 512 at batch 16 needs 1 KiB + 4 * 4125 * 16 * 16 * 4 bytes > 16 MiB."""
    M, K = 66000, 512
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 8, size=(M, K)).astype(np.uint8)
    from oracle import pack
    f = {"M": M, "K": K, "bits": 3, "fmt": "uniform", "group": 16, "codes_packed": pack.pack_bitstream(codes, 3),
         "scales": np.full((M, K // 16), 0.01, np.float16), "zeros": np.full((M, K // 16), 3, np.float16),
         "row_ptr": np.zeros(M + 1, np.int32), "col_idx": np.zeros(0, np.int32), "values": np.zeros(0, np.float16)}
    plan = qgemv.QGemv(f)
    x = torch.zeros((16, K), dtype=torch.float16, device="cuda")
    y = torch.zeros((16, M), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    say(f"[gpu] no-alloc refusal M={M} K={K} B=16")
    assert qgemv.lib().qgemv_run_noalloc(plan._h, x.data_ptr(), y.data_ptr(), 16, s) == -6
    assert qgemv.lib().qgemv_error_string(-6).startswith(b"workspace needed exceeds")
    plan.run(x, y)  # qgemv_run allocates the plan's workspace instead
    torch.cuda.synchronize()
    assert torch.all(y == 0).item()
    plan.close()
