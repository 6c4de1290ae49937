"""Benchmark of the dense-and-sparse quantized GEMV on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--batch B] [--no-cpu]

One step is one pass of the whole path over one batch: for every layer of
the workload, one qgemv_run -- decode of every packed code, the product with
x, the CSR outlier product into the same y, y written once.  Inputs are
synthetic arrays in the storage format with the workload's shapes, code
widths, FP16 tables and outlier structure, resident in HBM before timing
starts.

Distinct copies of each weight blob (>= 1 GiB in total) are cycled, launch i
reading copy i mod copies, and the timed replay starts at copy `steps`,
after the warm-up's copies, so every step streams its weights from HBM
rather than from the 256 MB last-level cache.  Each layer's timed region is one
HIP-graph replay of exactly K launches, bracketed by device synchronisation
and timed with HIP events recorded on the launch stream.

Prints ONE JSON line.  `value` is effective GB/s: algorithmic bytes per step
(packed codes, FP16 statistics or tables, CSR as FP16 value + int32 column +
int32 row pointer, x, y; each counted once) divided by the mean step time.
With the default workload the line also carries `targets`: both batch-1
shapes that have a 70 %-of-8-TB/s target (28672x8192 LUT-4 and 11008x4096
LUT-3), each next to a plain streaming read of the same number of bytes.

--copy-mb N also times a plain elementwise copy of N MiB (a kernel of known
traffic, used to calibrate the HBM byte counters of a profiler run).
--trace-summary CSV prints median / p10 / p90 of the timed replays' launches
in a rocprofv3 kernel trace (--output-format csv) of a bench.py run given the
same --steps and --warmup.
--counter-summary FETCH_CSV WRITE_CSV turns two rocprofv3 counter runs
(--pmc FETCH_SIZE, then --pmc WRITE_SIZE, each of a bench.py run with
--copy-mb N) into the HBM bytes per launch of the path's kernel, calibrated
on the copy kernel; --layer NAME limits a multi-layer workload to one layer.
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

# The CPU baseline runs on every host thread this process may use; the BLAS
# reads its thread count when numpy is first imported, so set it here (an
# existing setting is kept).
HOST_THREADS = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
    os.environ.setdefault(_v, str(HOST_THREADS))

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


def traffic_file(workload: str, batch: int, layer: str | None = None) -> str:
    tail = f"_{layer}" if layer else ""
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_b{batch}{tail}.json")


def load_traffic(workload: str, batch: int, src_hash: str, only_layer: str | None = None):
    """HBM bytes per step from committed rocprofv3 counter runs, if taken on this kernel source.

    A multi-layer workload has one file per distinct layer shape, named for
    the first layer of that shape; the step's traffic is their sum over the
    layers (None if any is missing or stale).
    """
    from synth import WORKLOADS
    wl = WORKLOADS[workload]
    if wl.layers:
        parts = []
        for name, M, K in wl.layers:
            if only_layer and name != only_layer:
                continue
            first = next(n for n, m, k in wl.layers if (m, k) == (M, K))
            parts.append(traffic_file(workload, batch, first))
    else:
        parts = [traffic_file(workload, batch)]
    total = 0
    for path in parts:
        if not os.path.exists(path):
            return None
        with open(path) as fh:
            t = json.load(fh)
        if t.get("kernel_src_sha") != src_hash:
            return None
        total += int(t["traffic_bytes_per_launch"])
    return total


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


# Layers of a block that read the same activations: in a decoder block q, k
# and v all take the normed hidden state, gate and up the normed attention
# output.  With --fuse each such group runs as one product over its stacked
# rows (one launch, x read once); the others run alone.
FUSED_GROUPS = {"block7b_u3": (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
                               ("down", ("down",)))}


def stack_rows(fs: list) -> dict:
    """One weight set whose rows are the rows of fs, in order (same K, format and code width).

    Every part of the storage format is per row (the code bitstream, the
    statistics or table, the CSR rows), so stacking is concatenation; the
    product over the stacked rows is the products of the parts, one after
    another in y.
    """
    import numpy as np
    f0 = fs[0]
    for f in fs[1:]:
        assert (f["K"], f["bits"], f["fmt"], f["group"]) == (f0["K"], f0["bits"], f0["fmt"], f0["group"])
    out = {k: f0[k] for k in ("K", "bits", "fmt", "group")}
    out["M"] = sum(f["M"] for f in fs)
    for key in ("codes_packed", "scales", "zeros", "lut", "coefs"):
        if key in f0:
            out[key] = np.concatenate([f[key] for f in fs], axis=0)
    base = np.cumsum([0] + [f["M"] for f in fs[:-1]])
    rows = np.concatenate([np.asarray(f["rows"], np.int64) + b for f, b in zip(fs, base)])
    cols = np.concatenate([np.asarray(f["cols"], np.int64) for f in fs])
    vals = np.concatenate([np.asarray(f["values"], np.float16) for f in fs])
    out["rows"], out["cols"] = rows, cols
    out["row_ptr"], out["col_idx"], out["values"] = csr_from_positions(out["M"], rows, cols, vals)
    return out


def launch_units(workload: str, fuse: bool):
    """(name, [(layer index, layer name), ...]) per launch of one step."""
    layers = workload_layers(workload)
    if not fuse or workload not in FUSED_GROUPS:
        return [(name, [(i, name)]) for i, name in layers]
    idx = {name: i for i, name in layers}
    return [(g, [(idx[n], n) for n in members]) for g, members in FUSED_GROUPS[workload]]


def host_description() -> dict:
    """CPU model and the BLAS build and thread count numpy runs on."""
    model = platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    b = blas[0] if blas else {}
    return {"cpu": model, "affinity_threads": HOST_THREADS,
            "blas": f"{b.get('internal_api', '?')} {b.get('version', '?')} ({b.get('architecture', '?')}, "
                    f"{b.get('threading_layer', '?')})",
            "blas_threads": int(b.get("num_threads", 1))}


def cpu_baseline(layers: list, alg_bytes: int, row_frac: float = 0.125, runs: int = 5):
    """The oracle's unpack + decode + GEMV + SpMV (y only) on the host cores.

    A seeded random 1/8 of every layer's rows, in row order; median of `runs`
    runs after one warm-up, scaled to all rows.
    """
    import numpy as np

    from oracle import gemv
    host = host_description()
    rng = np.random.default_rng(7)
    t_step, sample = 0.0, []
    for f, x16 in layers:
        M = f["M"]
        n = max(1, int(round(M * row_frac)))
        rows = np.sort(rng.choice(M, size=n, replace=False))
        chunk = max(1, (1 << 28) // (8 * f["K"]))

        def once():
            for r0 in range(0, n, chunk):
                gemv.gemv_rows(f, x16, rows[r0:r0 + chunk], scale=False)
        once()
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            once()
            ts.append(time.perf_counter() - t0)
        t_step += float(np.median(ts)) * M / n
        sample.append(f"{n}/{M} rows")
    return {
        "value": alg_bytes / t_step / 1e9,
        "unit": "GB/s",
        "us_per_step": t_step * 1e6,
        "cores": host["blas_threads"],
        "kind": "oracle",
        "sample": f"seeded random rows per layer ({', '.join(sample)}), decode + y in fp64 numpy; median of "
                  f"{runs} runs after 1 warm-up, scaled to all rows. BLAS products on {host['blas_threads']} "
                  f"threads; the unpack and decode steps are single-threaded numpy",
        "host": host,
    }


def time_graph(torch, launch, steps, warmup, stream, use_graph=True):
    """Mean ms per launch over `steps` launches, HIP events recorded on `stream`.

    launch(i) must read weight copy i mod copies.  Warm-up: `warmup` eager
    launches and one replay of a graph of launches 0 .. steps-1.  The timed
    region replays a second graph of launches steps .. 2*steps-1, so with at
    least 2*steps copies it reads only copies the warm-up has not touched,
    and with fewer it cycles through all of them (>= 1 GiB between two reads
    of one copy): either way the weights come from HBM, not from the 256 MB
    last-level cache.
    """
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i % steps)
    torch.cuda.synchronize()
    if use_graph:
        graphs = []
        for base in (0, steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    launch(base + i)
            graphs.append(g)
        torch.cuda.synchronize()
        graphs[0].replay()  # warm-up replay (untimed)
        torch.cuda.synchronize()
    else:
        with torch.cuda.stream(stream):
            for i in range(steps):
                launch(i)
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        if use_graph:
            graphs[1].replay()
        else:
            for i in range(steps):
                launch(steps + i)
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def measure(torch, qgemv, workload, B, steps, warmup, rotate_gib, stream, dev, use_graph, only_layer=None,
            fuse=False):
    """Per-launch timing of one workload; returns (per_layer, alg_total, ms_total, cpu_layers).

    Without fuse every layer is one launch; with fuse the layers of a
    FUSED_GROUPS entry run as one launch over their stacked rows, with the
    group's first layer's x.
    """
    import numpy as np

    from synth import make_x
    per_layer, cpu_layers = [], []
    alg_total, ms_total = 0, 0.0
    for lname, members in launch_units(workload, fuse):
        if only_layer and lname != only_layer:
            continue
        layer = members[0][0]
        parts = [format_inputs(workload, i) for i, _ in members]
        f = parts[0] if len(parts) == 1 else stack_rows(parts)
        M, K = f["M"], f["K"]
        host_blob = qgemv.repack(f)
        # distinct copies whose total is >= rotate_gib; launch i reads copy i % copies
        copies = max(1, min(512, math.ceil(rotate_gib * (1 << 30) / host_blob.size)))
        plans = [qgemv.QGemv(f, device="cuda:0", blob=host_blob) for _ in range(copies)]
        x16 = make_x(workload, B, K, layer, parts[0]["M"])
        x = torch.from_numpy(x16).to(dev)
        ys = [torch.empty((B, M), dtype=torch.float32, device=dev) for _ in range(copies)]
        torch.cuda.synchronize()

        def launch(i):
            plans[i % copies].run(x, ys[i % copies], stream=stream)

        # every copy runs once eagerly before capture (a plan's first batched
        # run allocates its workspace, which cannot happen under capture)
        with torch.cuda.stream(stream):
            for i in range(copies):
                launch(i)
        torch.cuda.synchronize()
        ms = time_graph(torch, launch, steps, warmup, stream, use_graph=use_graph)
        # every copy that ran must have produced the same, finite y
        y0 = ys[0].cpu().numpy()
        assert np.all(np.isfinite(y0)), f"{lname}: non-finite output"
        for y in ys[1:min(copies, 2 * steps)]:
            assert np.array_equal(y.cpu().numpy(), y0), f"{lname}: copies disagree"
        alg = algorithmic_bytes(f, B)
        alg_total += alg
        ms_total += ms
        per_layer.append({"layer": lname, "M": M, "K": K, "nnz": int(f["row_ptr"][-1]), "us": round(ms * 1e3, 3),
                          "GBs": round(alg / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": alg,
                          "weight_copies_rotated": copies,
                          "distinct_blob_bytes_per_replay": int(min(steps, copies) * host_blob.size),
                          "timed_copies_untouched_by_warmup": copies >= 2 * steps})
        cpu_layers.append((f, x16))
        del plans, ys
        torch.cuda.empty_cache()
    return per_layer, alg_total, ms_total, cpu_layers


def read_floor(torch, qgemv, nbytes, steps, warmup, stream, dev):
    """µs of one plain streaming read of nbytes (the library's read probe over
    distinct windows of a 2 GiB buffer, one graph replay)."""
    w = int(nbytes) // 16 * 16
    big = torch.full((2 << 30,), 7, dtype=torch.uint8, device=dev)
    nwin = (2 << 30) // w
    sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    ms = time_graph(torch, lambda i: qgemv.read_probe(big[(i % nwin) * w:(i % nwin + 1) * w], sink, stream=stream),
                    steps, warmup, stream)
    del big, sink
    torch.cuda.empty_cache()
    return ms * 1e3


PATH_KERNELS = ("k_pair", "k_stream", "k_xlds", "k_split", "k_huff")


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, batch: int, layer: str | None,
                       copy_mb: int) -> dict:
    """HBM bytes per launch of the path's kernel from two rocprofv3 counter runs.

    Each CSV holds one counter (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) for
    every dispatch of a bench.py run with --copy-mb copy_mb.  The path's
    kernel reads and writes the same bytes on every launch, so its value is
    the median over its dispatches; each counter is scaled by what it reads
    for the elementwise copy (copy_mb MiB read, copy_mb MiB written).
    """
    import csv

    import numpy as np

    def per_dispatch(path):
        vals, names = {}, {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                d = int(r["Dispatch_Id"])
                vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
                names[d] = r["Kernel_Name"]
        return vals, names

    out = {"workload": workload, "batch": batch}
    if layer:
        out["layer"] = layer
    res = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        vals, names = per_dispatch(path)
        ours = [v for d, v in vals.items() if any(k in names[d] for k in PATH_KERNELS)]
        cal = [v for d, v in vals.items() if "MulFunctor" in names[d]]
        kern = sorted({names[d].split("(unsigned")[0].replace("void ", "").replace("(anonymous namespace)::", "")
                       for d in vals if any(k in names[d] for k in PATH_KERNELS)})
        if not ours or not cal:
            raise SystemExit(f"{path}: no dispatches of the path's kernels or of the calibration copy")
        res[key] = (float(np.median(ours)), len(ours), float(np.median(cal)), kern)
    copy_kib = copy_mb * 1024.0
    f_kib, n, f_cal, kern = res["fetch"]
    w_kib, _, w_cal, _ = res["write"]
    f_scale, w_scale = copy_kib / f_cal, copy_kib / w_cal
    traffic = f_kib * f_scale * 1024 + w_kib * w_scale * 1024
    fi = format_inputs(workload, next(i for i, nm in workload_layers(workload) if layer in (None, nm)))
    alg = algorithmic_bytes(fi, batch)
    out.update({"kernels": kern, "kernel_src_sha": kernel_source_hash(),
                "traffic_bytes_per_launch": int(round(traffic)),
                "fetch_kib_per_dispatch": round(f_kib, 3), "write_kib_per_dispatch": round(w_kib, 3),
                "dispatches": n, "copy_fetch_kib": f_cal, "copy_write_kib": w_cal,
                "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
                "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round(traffic / alg, 4)})
    return out


def counter_table(path: str) -> str:
    """Per kernel of a rocprofv3 counter run (csv): dispatches and the median of each counter per dispatch."""
    import csv

    import numpy as np
    per = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per.setdefault(key, {})
            per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (d, name), cs in per.items():
        if any(k in name for k in PATH_KERNELS):
            short = name.split("(unsigned")[0].replace("void ", "").replace("(anonymous namespace)::", "")
            by_kernel.setdefault(short, []).append(cs)
    counters = sorted({c for cs in per.values() for c in cs})
    out = ["kernel | dispatches | " + " | ".join(counters)]
    for k, lst in sorted(by_kernel.items()):
        med = [float(np.median([cs.get(c, 0.0) for cs in lst])) for c in counters]
        out.append(f"{k} | {len(lst)} | " + " | ".join(f"{v:.6g}" for v in med))
    return "\n".join(out)


def summarize_trace(path: str, steps: int, warmup: int) -> str:
    """Per-launch durations of the timed replays in a rocprofv3 kernel trace.

    For each layer bench.py dispatches the layer's kernel `warmup` times
    eagerly, then replays two graphs of `steps` launches each (warm-up, then
    timed); graph capture and the checks between layers dispatch other
    kernels.  So a run of 2*steps (or warmup + 2*steps) consecutive dispatches
    of one of the path's kernels ends with a timed replay: its last `steps`
    dispatches.  Prints median, p10, p90 and mean per timed replay, in µs.
    """
    import csv

    import numpy as np
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    ours = lambda n: any(k in n for k in PATH_KERNELS)
    runs = []
    for t0, t1, name in rows:
        if runs and runs[-1][0] == name:
            runs[-1][1].append(t1 - t0)
        else:
            runs.append((name, [t1 - t0]))
    out = [f"timed replays in {os.path.basename(path)} ({steps} launches each, after {warmup} eager warm-up "
           f"launches and one warm-up replay; durations in us)",
           "kernel | launches | median | p10 | p90 | mean"]
    for name, d in runs:
        if not ours(name) or len(d) not in (2 * steps, warmup + 2 * steps):
            continue
        t = np.asarray(d[-steps:], dtype=np.float64) / 1e3
        short = name.split("(unsigned")[0].replace("void ", "").replace("(anonymous namespace)::", "")
        out.append(f"{short} | {len(t)} | {np.median(t):.3f} | {np.percentile(t, 10):.3f} | "
                   f"{np.percentile(t, 90):.3f} | {t.mean():.3f}")
    return "\n".join(out)


TARGETS = ("mlp70b_lut4", "mlp7b_lut3")  # the two batch-1 shapes with a 70 % of 8 TB/s target


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
    ap.add_argument("--no-targets", action="store_true",
                    help="skip the second target shape and the per-shape read floors")
    ap.add_argument("--copy-mb", type=int, default=0, help="also time a plain device copy of this many MiB")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured streaming-read ceiling")
    ap.add_argument("--read-probe-mb", type=float, default=0.0,
                    help="only time the read probe over windows of this many MB (rotated through 2 GiB)")
    ap.add_argument("--trace-summary", default=None, metavar="CSV",
                    help="only summarise the timed replays of a rocprofv3 kernel_trace.csv (no GPU)")
    ap.add_argument("--layer", default=None, help="only this layer (or fused group) of a multi-layer workload")
    ap.add_argument("--fuse", action="store_true",
                    help="run the layers that share x (q,k,v; gate,up) as one product over their stacked rows")
    ap.add_argument("--counter-table", default=None, metavar="CSV",
                    help="only print per-kernel median counters of a rocprofv3 counter run (no GPU)")
    ap.add_argument("--counter-summary", nargs=2, default=None, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="only turn two rocprofv3 counter runs into HBM bytes per launch (no GPU)")
    a = ap.parse_args()

    if a.trace_summary is not None:
        print(summarize_trace(a.trace_summary, a.steps, a.warmup))
        return
    if a.counter_table is not None:
        print(counter_table(a.counter_table))
        return
    if a.counter_summary is not None:
        B = a.batch or DEFAULT_BATCH.get(a.workload, 1)
        print(json.dumps(summarize_counters(a.counter_summary[0], a.counter_summary[1], a.workload, B, a.layer,
                                            a.copy_mb or 1024), indent=1))
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from dense_sparse_bit_amd import qgemv

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B = a.batch or DEFAULT_BATCH.get(a.workload, 1)
    stream = torch.cuda.Stream(device=dev)

    if a.read_probe_mb:
        us = read_floor(torch, qgemv, a.read_probe_mb * 1e6, a.steps, a.warmup, stream, dev)
        w = int(a.read_probe_mb * 1e6) // 16 * 16
        print(json.dumps({"read_probe": {"bytes": w, "us": round(us, 3), "GBs": round(w / (us * 1e-6) / 1e9, 1)}}),
              flush=True)
        return

    per_layer, alg_total, ms_total, cpu_layers = measure(torch, qgemv, a.workload, B, a.steps, a.warmup,
                                                         a.rotate_gib, stream, dev, not a.no_graph, a.layer, a.fuse)
    if not per_layer:
        raise SystemExit(f"{a.workload} has no layer {a.layer!r}")
    us = ms_total * 1e3
    gbs = alg_total / (ms_total * 1e-3) / 1e9
    flops = sum(2.0 * B * p["M"] * p["K"] for p in per_layer)
    src = kernel_source_hash()
    traffic = None if a.fuse else load_traffic(a.workload, B, src, a.layer)
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
        "config": {"workload": f"{a.workload}: {WORKLOAD_NOTES[a.workload]}, batch {B}" +
                               ("; q,k,v and gate,up each one product over their stacked rows (shared x)"
                                if a.fuse and a.workload in FUSED_GROUPS else ""), "batch": B,
                   "bits": first.get("bits", 0), "format": first["fmt"], "layers": per_layer,
                   "timing": ("eager launches" if a.no_graph else "one HIP-graph replay of all steps per layer") +
                             ", HIP events on the launch stream; the timed replay reads weight copies the "
                             "warm-up did not touch (or cycles through >= 1 GiB of them)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_step": alg_total, "kernel_src_sha": src},
    }
    if B > 1:
        tf = flops / (ms_total * 1e-3) / 1e12
        out["mfma"] = {"tflops": round(tf, 2), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                       "util": round(tf / MFMA_F16_PEAK_TFLOPS, 5),
                       "note": "dense flops 2*B*M*K at fp16 MFMA peak; the path stays HBM-bound"}
    if not a.no_targets and B == 1 and a.workload in TARGETS:
        # both 70 %-target shapes at batch 1, each next to a plain read of its bytes
        targets = []
        for wname in TARGETS:
            if wname == a.workload:
                t_us, t_alg = us, alg_total
            else:
                pl, t_alg, t_ms, _ = measure(torch, qgemv, wname, 1, a.steps, a.warmup, a.rotate_gib, stream, dev,
                                             not a.no_graph)
                t_us = t_ms * 1e3
            floor_us = read_floor(torch, qgemv, t_alg, a.steps, a.warmup, stream, dev)
            targets.append({"workload": wname, "us": round(t_us, 3), "GBs": round(t_alg / (t_us * 1e-6) / 1e9, 1),
                            "frac_of_8TBs": round(t_alg / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "target_us_at_70pct": round(t_alg / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6, 3),
                            "plain_read_us_same_bytes": round(floor_us, 3),
                            "frac_of_plain_read": round(floor_us / t_us, 4)})
        out["targets"] = targets
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
