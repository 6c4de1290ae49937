"""Benchmark of the dense-and-sparse quantized GEMV on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--batch B] [--no-cpu]

One step is one pass of the whole path over one batch: for every layer of
the workload, one qgemv_run -- decode of every packed code, the product with
x, the CSR outlier product into the same y, y written once.  Inputs are
synthetic arrays in the storage format with the workload's shapes, code
widths, FP16 tables and outlier structure, resident in HBM before timing
starts.

Distinct copies of each weight blob (>= 1 GiB in total) are cycled so that
every step streams its weights from HBM rather than from the 256 MB
last-level cache.  Each layer's timed region is one HIP-graph replay of
exactly K launches, bracketed by device synchronisation and timed with HIP
events recorded on the launch stream.

Prints ONE JSON line.  `value` is effective GB/s: algorithmic bytes per step
(packed codes, FP16 statistics or tables, CSR as FP16 value + int32 column +
int32 row pointer, x, y; each counted once) divided by the mean step time.

--copy-mb N also times a plain elementwise copy of N MiB (a kernel of known
traffic, used to calibrate the HBM byte counters of a profiler run).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

WORKLOAD_NOTES = {
    "mlp70b_lut4": "70B-shaped MLP 28672x8192, 4-bit codes + per-row FP16 LUT-16, 0.5% FP16 CSR outliers "
                   "(5% of rows at 10x density + 2 full columns)",
    "mlp7b_lut3": "MLP up-proj 11008x4096, 3-bit codes + per-row FP16 LUT-8, 0.45% FP16 CSR outliers",
    "attn7b_u3": "attention projection 4096x4096, 3-bit codes + FP16 scale/zero per 16, 0.5% FP16 CSR outliers",
    "tiny_u4": "512x512, 4-bit codes + FP16 scale/zero per 16, 1% FP16 CSR outliers",
    "block7b_u3": "7B decoder block q,k,v,o 4096x4096, gate,up 11008x4096, down 4096x11008; 3-bit codes + "
                  "FP16 scale/zero per 16, 1% FP16 CSR outliers",
    "mlp7b_bpdq3": "MLP up-proj 11008x4096, 3-bit BPDQ codes + 4 FP16 bit-plane coefficients per row and group of "
                   "64, 0.45% FP16 CSR outliers",
    "mlp7b_hptq": "MLP up-proj 11008x4096, HPTQ prefix-coded integers (about 3.2 bits per weight) on one grid with "
                  "an FP16 step per row and group of 128, 0.45% outliers on the same grid",
}
DEFAULT_BATCH = {"block7b_u3": 16}


def algorithmic_bytes(f: dict, B: int = 1) -> int:
    M, K, bits = f["M"], f["K"], f.get("bits", 0)
    nnz = int(f["row_ptr"][-1])
    if f["fmt"] == "hptq":  # stream, steps, row starts, the code's integers and lengths, x, y
        return (int(f["row_bits"][-1]) + 7) // 8 + M * (K // f["group"]) * 2 + 8 * (M + 1) + \
            3 * len(f["huff_sym"]) + 2 * B * K + 4 * B * M
    codes = M * K * bits // 8
    if f["fmt"] == "uniform":
        meta = M * (K // 16) * 4
    elif f["fmt"] == "bpdq":
        meta = M * (K // f["group"]) * (bits + 1) * 2
    else:
        meta = M * (1 << bits) * 2
    csr = 6 * nnz + 4 * (M + 1)
    return codes + meta + csr + 2 * B * K + 4 * B * M


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "dense_sparse_bit_amd", "csrc")
    for n in sorted(os.listdir(d)):
        with open(os.path.join(d, n), "rb") as fh:
            h.update(n.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, batch: int, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_b{batch}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_src_sha") != src_hash:
        return None
    return t.get("traffic_bytes_per_launch")


def csr_from_positions(M, rows, cols, values):
    import numpy as np
    counts = np.bincount(rows, minlength=M)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_ptr, cols.astype(np.int32), np.asarray(values, dtype=np.float16)


def format_inputs(workload: str, layer: int = 0):
    from synth import make_format_inputs
    f = make_format_inputs(workload, layer)
    f["row_ptr"], f["col_idx"], f["values"] = csr_from_positions(f["M"], f["rows"], f["cols"], f["values"])
    return f


def workload_layers(workload: str):
    from synth import WORKLOADS
    wl = WORKLOADS[workload]
    if wl.layers:
        return [(i, name) for i, (name, _, _) in enumerate(wl.layers)]
    return [(0, "w")]


def cpu_baseline(layers: list, alg_bytes: int, target_s: float = 12.0):
    """The oracle's unpack + decode + GEMV + SpMV, single thread, on a bounded row sample of every layer."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import gemv
    rng = np.random.default_rng(7)
    budget = target_s / len(layers)
    t_step, sample = 0.0, []
    with threadpool_limits(limits=1):
        for f, x16 in layers:
            M = f["M"]
            n = min(M, max(64, 1024 // len(layers)))
            rows = np.sort(rng.choice(M, size=n, replace=False))
            t0 = time.perf_counter()
            gemv.gemv_rows(f, x16, rows)
            one = time.perf_counter() - t0
            reps = max(1, min(20, int(budget / max(one, 1e-3))))
            ts = []
            for _ in range(reps):
                t0 = time.perf_counter()
                gemv.gemv_rows(f, x16, rows)
                ts.append(time.perf_counter() - t0)
            t_step += float(np.median(ts)) * M / n
            sample.append(f"{n}/{M} rows x{reps}")
    return {
        "value": alg_bytes / t_step / 1e9,
        "unit": "GB/s",
        "us_per_step": t_step * 1e6,
        "cores": 1,
        "kind": "oracle",
        "sample": f"random rows (seed 7) per layer: {', '.join(sample)}; median run after 1 warm-up, scaled to "
                  f"all rows; fp64 numpy, 1 thread; host CPU: {platform.processor() or platform.machine()}",
    }


def time_graph(torch, launch, steps, warmup, stream, use_graph=True):
    """Mean ms per launch of `launch(i)` over `steps` launches (one graph replay), HIP events on `stream`."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                launch(i)
        torch.cuda.synchronize()
        graph.replay()  # warm the graph once (untimed)
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                launch(i)
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="mlp70b_lut4", choices=sorted(WORKLOAD_NOTES))
    ap.add_argument("--batch", type=int, default=None, choices=[1, 8, 16])
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--copy-mb", type=int, default=0, help="also time a plain device copy of this many MiB")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured streaming-read ceiling")
    ap.add_argument("--read-probe-mb", type=float, default=0.0,
                    help="only time the read probe over windows of this many MB (rotated through 2 GiB)")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from dense_sparse_bit_amd import qgemv
    from synth import make_x

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B = a.batch or DEFAULT_BATCH.get(a.workload, 1)
    stream = torch.cuda.Stream(device=dev)

    if a.read_probe_mb:
        # Plain streaming reads of one layer's size: distinct windows of a
        # 2 GiB buffer, so every launch reads from HBM, one HIP-graph replay.
        w = int(a.read_probe_mb * 1e6) // 16 * 16
        big = torch.full((2 << 30,), 7, dtype=torch.uint8, device=dev)
        nwin = (2 << 30) // w
        sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
        ms_p = time_graph(torch, lambda i: qgemv.read_probe(big[(i % nwin) * w:(i % nwin + 1) * w], sink,
                                                             stream=stream), a.steps, a.warmup, stream)
        print(json.dumps({"read_probe": {"bytes": w, "us": round(ms_p * 1e3, 3),
                                         "GBs": round(w / (ms_p * 1e-3) / 1e9, 1), "windows": nwin}}), flush=True)
        return

    per_layer, cpu_layers = [], []
    alg_total, ms_total = 0, 0.0
    for layer, lname in workload_layers(a.workload):
        f = format_inputs(a.workload, layer)
        M, K = f["M"], f["K"]
        host_blob = qgemv.repack(f)
        copies = max(1, min(a.steps, 256, math.ceil(a.rotate_gib * (1 << 30) / host_blob.size)))
        plans = [qgemv.QGemv(f, device="cuda:0", blob=host_blob) for _ in range(copies)]
        x16 = make_x(a.workload, B, K, layer, M)
        x = torch.from_numpy(x16).to(dev)
        ys = [torch.empty((B, M), dtype=torch.float32, device=dev) for _ in range(copies)]
        torch.cuda.synchronize()

        def launch(i):
            plans[i % copies].run(x, ys[i % copies], stream=stream)

        ms = time_graph(torch, launch, a.steps, a.warmup, stream, use_graph=not a.no_graph)
        # every copy must have produced the same, finite y
        y0 = ys[0].cpu().numpy()
        assert np.all(np.isfinite(y0)), f"{lname}: non-finite output"
        for y in ys[1:]:
            assert np.array_equal(y.cpu().numpy(), y0), f"{lname}: copies disagree"
        alg = algorithmic_bytes(f, B)
        alg_total += alg
        ms_total += ms
        per_layer.append({"layer": lname, "M": M, "K": K, "nnz": int(f["row_ptr"][-1]), "us": round(ms * 1e3, 3),
                          "GBs": round(alg / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": alg,
                          "weight_copies_rotated": copies})
        cpu_layers.append((f, x16))
        del plans, ys
        torch.cuda.empty_cache()

    us = ms_total * 1e3
    gbs = alg_total / (ms_total * 1e-3) / 1e9
    flops = sum(2.0 * B * p["M"] * p["K"] for p in per_layer)
    src = kernel_source_hash()
    traffic = load_traffic(a.workload, B, src)
    first = cpu_layers[0][0]
    out = {
        "metric": "µs/layer and effective GB/s (batch-1 qGEMV) as % of MI355X HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "us_per_layer": round(us / len(per_layer), 3),
        "us_per_step": round(us, 3),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_total, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"{a.workload}: {WORKLOAD_NOTES[a.workload]}, batch {B}", "batch": B,
                   "bits": first.get("bits", 0), "format": first["fmt"], "layers": per_layer,
                   "timing": "eager launches" if a.no_graph else "one HIP-graph replay of all steps per layer"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_step": alg_total, "kernel_src_sha": src},
    }
    if B > 1:
        tf = flops / (ms_total * 1e-3) / 1e12
        out["mfma"] = {"tflops": round(tf, 2), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                       "util": round(tf / MFMA_F16_PEAK_TFLOPS, 5),
                       "note": "dense flops 2*B*M*K at fp16 MFMA peak; the path stays HBM-bound"}
    if not a.no_ceiling:
        # The streaming-read rate of this GPU, measured in the same run: the
        # library's read probe (16-byte non-temporal loads) over 1 GiB.
        n = 1 << 30
        buf = torch.full((n,), 7, dtype=torch.uint8, device=dev)
        sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
        ms_r = time_graph(torch, lambda i: qgemv.read_probe(buf, sink, stream=stream), 20, 3, stream,
                          use_graph=False)
        ceil_gbs = n / (ms_r * 1e-3) / 1e9
        out["roofline"]["measured_read_ceiling"] = {"GBs": round(ceil_gbs, 1), "frac": round(gbs / ceil_gbs, 4),
                                                    "kernel": "qgemv_read_probe over 1 GiB, eager"}
        del buf, sink
    if a.copy_mb:
        n = a.copy_mb << 20
        src_t = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst_t = torch.empty(n // 4, dtype=torch.float32, device=dev)
        # an elementwise kernel that reads n bytes and writes n bytes
        ms_copy = time_graph(torch, lambda i: torch.mul(src_t, 1.0, out=dst_t), 20, 3, stream)
        out["copy_calibration"] = {"bytes_read": n, "bytes_written": n, "us": round(ms_copy * 1e3, 3),
                                   "GBs_read_plus_write": round(2 * n / (ms_copy * 1e-3) / 1e9, 1)}
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cpu_layers, alg_total)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
