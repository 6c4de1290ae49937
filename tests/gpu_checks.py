"""Helpers of the GPU parity tests (not collected): runs framed by canaries,
and all-row / all-code comparisons against the oracle in row chunks."""

import sys

import numpy as np

from oracle import gemv, pack

CANARY = np.int32(0x7FC0DEAD)  # a NaN bit pattern no kernel writes
PAD = 256                      # canary words on each side (16-byte multiple)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _framed(torch, n, dtype, device, fill):
    """A flat buffer of PAD + n + PAD elements; the middle n are filled with `fill`,
    the pads with CANARY words.  Returns (buffer, view of the middle)."""
    itemsize = torch.tensor([], dtype=dtype).element_size()
    pad = PAD * 4 // itemsize
    buf = torch.empty(pad * 2 + n, dtype=dtype, device=device)
    buf.view(torch.int32 if itemsize == 4 else torch.uint8).fill_(int(CANARY) if itemsize == 4 else 0xA5)
    mid = buf[pad:pad + n]
    mid.fill_(fill)
    return buf, mid, pad


def _check_pads(buf, pad, what):
    import torch
    v = buf.view(torch.int32) if buf.element_size() == 4 else buf
    want = int(CANARY) if buf.element_size() == 4 else 0xA5
    head, tail = v[:pad].cpu().numpy(), v[-pad:].cpu().numpy()
    assert np.all(head == want) and np.all(tail == want), f"{what}: a write landed outside the output"


def run_framed(torch, plan, x16):
    """y [B, M] of plan.run on the rows of x16, in a NaN-filled output framed by
    canary words; checks that every output was written and nothing outside."""
    x = torch.from_numpy(np.ascontiguousarray(x16)).cuda()
    B = x16.shape[0]
    buf, mid, pad = _framed(torch, B * plan.M, torch.float32, "cuda", float("nan"))
    y = mid.view(B, plan.M)
    plan.run(x, y)
    torch.cuda.synchronize()
    _check_pads(buf, pad, "y")
    out = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out)), "output not fully written"
    return out


def unpack_framed(torch, plan):
    """Codes [M, K] of qgemv_debug_unpack into a framed buffer."""
    from dense_sparse_bit_amd import qgemv
    buf, mid, pad = _framed(torch, plan.M * plan.K, torch.uint8, "cuda", 0xFF)
    s = torch.cuda.current_stream().cuda_stream
    st = qgemv.lib().qgemv_debug_unpack(plan._h, mid.data_ptr(), s)
    assert st == 0, f"qgemv_debug_unpack: {st}"
    torch.cuda.synchronize()
    _check_pads(buf, pad, "codes")
    return mid.view(plan.M, plan.K).cpu().numpy()


def check_codes_all(codes_gpu, enc, chunk=2048):
    """Every code equals the canonical bitstream's (or the encoder's unpacked codes)."""
    M, K = enc["M"], enc["K"]
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        if enc.get("codes") is not None:
            ref = np.asarray(enc["codes"][r0:r1])
        else:
            ref = pack.unpack_bitstream(np.asarray(enc["codes_packed"])[r0:r1], enc["bits"], K)
        if not np.array_equal(codes_gpu[r0:r1], ref):
            bad = np.argwhere(codes_gpu[r0:r1] != ref)[0]
            raise AssertionError(f"code mismatch at row {r0 + bad[0]}, column {bad[1]}")


def check_y_all(y_gpu, enc, x16, chunk=None):
    """|y_gpu - y| <= 1e-4 A + 1e-6 for every output, the oracle run in row chunks."""
    M, K = enc["M"], enc["K"]
    chunk = chunk or max(1, (1 << 28) // (8 * K))  # about 256 MB of fp64 weights per chunk
    worst = 0.0
    for r0 in range(0, M, chunk):
        rows = np.arange(r0, min(M, r0 + chunk))
        y_ref, A = gemv.gemv_rows(enc, x16[:y_gpu.shape[0]], rows)
        ok, w = gemv.within_tolerance(y_gpu[:, rows], y_ref, A)
        assert ok, f"rows {rows[0]}..{rows[-1]}: tolerance exceeded, worst |dy|/(1e-4 A + 1e-6) = {w:.3f}"
        worst = max(worst, w)
    return worst


def check_all(codes_gpu, runs, enc, chunk=None):
    """Codes and outputs of every row against the oracle, in row chunks.

    codes_gpu: [M, K] uint8 from qgemv_debug_unpack (or None to skip codes);
    runs: list of (y_gpu [B, M], x16 [B, K]).  Each chunk's codes are unpacked
    once from the canonical bytes and decoded once for all runs.
    Returns the worst |dy| / (1e-4 A + 1e-6) over all outputs.
    """
    M, K = enc["M"], enc["K"]
    chunk = chunk or max(1, (1 << 28) // (8 * K))
    worst = 0.0
    for r0 in range(0, M, chunk):
        rows = np.arange(r0, min(M, r0 + chunk))
        if enc.get("codes") is not None:
            ref = np.asarray(enc["codes"][r0:rows[-1] + 1])
        else:
            ref = pack.unpack_bitstream(np.asarray(enc["codes_packed"])[r0:rows[-1] + 1], enc["bits"], K)
        if codes_gpu is not None and not np.array_equal(codes_gpu[r0:rows[-1] + 1], ref):
            bad = np.argwhere(codes_gpu[r0:rows[-1] + 1] != ref)[0]
            raise AssertionError(f"code mismatch at row {r0 + bad[0]}, column {bad[1]}")
        D = gemv.decode_rows(enc, rows, codes=ref)
        for y_gpu, x16 in runs:
            y_ref, A = gemv.gemv_rows(enc, x16, rows, D=D)
            ok, w = gemv.within_tolerance(y_gpu[:, rows], y_ref, A)
            assert ok, (f"B={x16.shape[0]} rows {rows[0]}..{rows[-1]}: tolerance exceeded, "
                        f"worst |dy|/(1e-4 A + 1e-6) = {w:.3f}")
            worst = max(worst, w)
    return worst
