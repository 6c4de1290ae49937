"""ctypes binding of libdsb_qgemv.so (argument marshalling only).

Every step of the product runs inside the library's HIP kernels; PyTorch is
used here only to own device memory and to name the current HIP stream.
If the shared library is missing this module raises instead of falling back
to anything else.

Canonical arrays are passed as a dict with the keys of the C struct
``qgemv_weights``: M, K, bits, fmt ("uniform" | "lut" | "bpdq"), group,
codes_packed (uint8 [M, K*bits/8]), scales / zeros (FP16 [M, K/16]), lut (FP16
[M, 2^bits]) or coefs (FP16 [M, K/group, bits+1]), row_ptr (int32 [M+1]),
col_idx (int32 [nnz]), values (FP16 [nnz]); "hptq" instead: stream (bytes),
row_bits (int64 [M+1]), huff_len (uint8), huff_sym (int16), scales (FP16
[M, K/128]).
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsb_qgemv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qgemv.h")

FMT = {"uniform": 0, "lut": 1, "bpdq": 2, "hptq": 3}
STATUS = {0: "QGEMV_OK", -1: "QGEMV_ERR_INVALID_ARG", -2: "QGEMV_ERR_MALFORMED_CSR",
          -3: "QGEMV_ERR_UNSUPPORTED", -4: "QGEMV_ERR_HIP", -5: "QGEMV_ERR_SIZE", -6: "QGEMV_ERR_SCRATCH"}



def read_probe(src, sink, stream=None):
    """Enqueue one non-temporal read of the device tensor `src` (its bytes) into
    per-thread XOR words in the int32/uint32 device tensor `sink`; measurement
    only (the streaming-read ceiling)."""
    import torch
    nbytes = src.numel() * src.element_size()
    s = (stream or torch.cuda.current_stream(src.device)).cuda_stream
    _check(lib().qgemv_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), s), "qgemv_read_probe")

class QgemvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")


class Weights(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int32), ("K", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("format", ctypes.c_int32), ("group_size", ctypes.c_int32), ("nnz", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
        ("lut", ctypes.c_void_p), ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
        ("values", ctypes.c_void_p), ("coefs", ctypes.c_void_p),
        ("huff_nsym", ctypes.c_int32), ("huff_len", ctypes.c_void_p), ("huff_sym", ctypes.c_void_p),
        ("row_bits", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m dense_sparse_bit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.qgemv_packed_size.argtypes = [P(Weights), P(ctypes.c_size_t)]
    L.qgemv_repack.argtypes = [P(Weights), ctypes.c_void_p, ctypes.c_size_t]
    L.qgemv_unpack_host.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t]
    L.qgemv_create.argtypes = [P(ctypes.c_void_p), P(Weights), ctypes.c_void_p, ctypes.c_size_t]
    L.qgemv_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.qgemv_run_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.c_void_p]
    L.qgemv_debug_unpack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.qgemv_destroy.argtypes = [ctypes.c_void_p]
    L.qgemv_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.qgemv_error_string.argtypes = [ctypes.c_int]
    L.qgemv_error_string.restype = ctypes.c_char_p
    L.qgemv_last_hip_error.argtypes = []
    for f in ("qgemv_packed_size", "qgemv_repack", "qgemv_unpack_host", "qgemv_create", "qgemv_run", "qgemv_run_noalloc",
              "qgemv_debug_unpack", "qgemv_read_probe", "qgemv_destroy", "qgemv_last_hip_error"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def header_symbols() -> list:
    """Names of the functions declared in include/qgemv.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qgemv_\w+)\s*\(", text, re.M)))


def _check(st: int, what: str):
    if st != 0:
        raise QgemvError(st, what)


def make_weights(w: dict):
    """Build the C descriptor; returns (struct, list of arrays that must stay alive)."""
    keep = []

    def ptr(a, dtype):
        if a is None:
            return None
        a = np.asarray(a)
        if dtype == np.uint16 and a.dtype == np.float16:
            a = a.view(np.uint16)
        a = np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a.ctypes.data

    fmt = FMT[w["fmt"]] if isinstance(w["fmt"], str) else int(w["fmt"])
    row_ptr = np.asarray(w["row_ptr"])
    nnz = int(row_ptr[-1]) if len(row_ptr) else 0
    s = Weights()
    s.M, s.K, s.bits, s.format = int(w["M"]), int(w["K"]), int(w.get("bits", 0)), fmt
    s.group_size = int(w.get("group", 16) or 16)
    s.nnz = int(w.get("nnz", nnz))
    s.codes = ptr(w["stream"] if fmt == FMT["hptq"] else w["codes_packed"], np.uint8)
    s.scales = ptr(w.get("scales"), np.uint16)
    s.zeros = ptr(w.get("zeros"), np.uint16)
    s.lut = ptr(w.get("lut"), np.uint16)
    s.row_ptr = ptr(row_ptr, np.int32)
    s.col_idx = ptr(w.get("col_idx"), np.int32) if nnz else None
    s.values = ptr(w.get("values"), np.uint16) if nnz else None
    s.coefs = ptr(w.get("coefs"), np.uint16)
    if w.get("huff_sym") is not None:  # HPTQ: the prefix code and the row starts in the stream
        s.huff_nsym = len(w["huff_sym"])
        s.huff_len = ptr(w["huff_len"], np.uint8)
        s.huff_sym = ptr(w["huff_sym"], np.int16)
        s.row_bits = ptr(w["row_bits"], np.int64)
        s.bits = 0
    return s, keep


def packed_size(w: dict) -> int:
    s, keep = make_weights(w)
    n = ctypes.c_size_t(0)
    _check(lib().qgemv_packed_size(ctypes.byref(s), ctypes.byref(n)), "qgemv_packed_size")
    return n.value


def repack(w: dict) -> np.ndarray:
    """Host repack into the gfx950 blob (uint8 array)."""
    s, keep = make_weights(w)
    n = ctypes.c_size_t(0)
    _check(lib().qgemv_packed_size(ctypes.byref(s), ctypes.byref(n)), "qgemv_packed_size")
    blob = np.zeros(n.value, dtype=np.uint8)
    _check(lib().qgemv_repack(ctypes.byref(s), blob.ctypes.data, n.value), "qgemv_repack")
    return blob


def unpack_host(blob: np.ndarray, M: int, K: int) -> np.ndarray:
    out = np.zeros((M, K), dtype=np.uint8)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    _check(lib().qgemv_unpack_host(blob.ctypes.data, blob.size, out.ctypes.data, out.size), "qgemv_unpack_host")
    return out


class QGemv:
    """A plan bound to one weight set in device memory (owned by a torch tensor)."""

    def __init__(self, w: dict, device: str = "cuda", blob: np.ndarray | None = None):
        import torch
        self.M, self.K = int(w["M"]), int(w["K"])
        self._desc, self._keep = make_weights(w)
        host = repack(w) if blob is None else blob
        self.blob_bytes = int(host.size)
        self.blob = torch.empty(self.blob_bytes, dtype=torch.uint8, device=device)
        self.blob.copy_(torch.from_numpy(host))
        torch.cuda.synchronize(self.blob.device)
        h = ctypes.c_void_p(0)
        _check(lib().qgemv_create(ctypes.byref(h), ctypes.byref(self._desc), self.blob.data_ptr(),
                                  self.blob_bytes), "qgemv_create")
        self._h = h

    def run(self, x, y=None, stream=None):
        """y[B, M] (fp32) = W x for x[B, K] (FP16, on the plan's device); returns y."""
        import torch
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.dtype != torch.float16 or not x.is_contiguous() or x.shape[1] != self.K:
            raise ValueError("x must be a contiguous FP16 [B, K] tensor")
        B = x.shape[0]
        if y is None:
            y = torch.empty((B, self.M), dtype=torch.float32, device=x.device)
        if y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (B, self.M):
            raise ValueError("y must be a contiguous fp32 [B, M] tensor")
        s = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        _check(lib().qgemv_run(self._h, x.data_ptr(), y.data_ptr(), B, s), "qgemv_run")
        return y

    def run_noalloc(self, x, y, stream=None):
        """As run(), into a given y, through qgemv_run_noalloc (no device allocation)."""
        import torch
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.dtype != torch.float16 or not x.is_contiguous() or x.shape[1] != self.K:
            raise ValueError("x must be a contiguous FP16 [B, K] tensor")
        B = x.shape[0]
        if y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (B, self.M):
            raise ValueError("y must be a contiguous fp32 [B, M] tensor")
        s = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        _check(lib().qgemv_run_noalloc(self._h, x.data_ptr(), y.data_ptr(), B, s), "qgemv_run_noalloc")
        return y

    def debug_unpack(self, stream=None):
        import torch
        out = torch.empty((self.M, self.K), dtype=torch.uint8, device=self.blob.device)
        s = (stream or torch.cuda.current_stream(self.blob.device)).cuda_stream
        _check(lib().qgemv_debug_unpack(self._h, out.data_ptr(), s), "qgemv_debug_unpack")
        return out

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().qgemv_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
