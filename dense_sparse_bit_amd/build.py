"""Build the HIP library libdsb_qgemv.so in-tree for gfx950.

    python -m dense_sparse_bit_amd.build            # build
    python -m dense_sparse_bit_amd.build --asm DIR  # also keep the gfx950 assembly in DIR
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsb_qgemv.so")
SOURCES = ["qgemv_kernels.hip", "qgemv_host.cpp"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed-FP32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, *srcs, "-o", tmp]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps"]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = asm_dir or CSRC
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for -save-temps output")
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.v, asm_dir=a.asm))


if __name__ == "__main__":
    main()
