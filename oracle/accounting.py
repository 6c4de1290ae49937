"""Bits-per-weight accounting -- test infrastructure only.

[SpQR] "Le format de stockage sparse": about 1 % of the entries at 16 bit plus
the index overhead cost roughly 0.5-1 extra bit per weight.
[SqLLM] "Bits / Formats supportés": about 3 bits dense plus about 0.1 bit per
weight sparse at about 0.45 % outliers.
"""

from __future__ import annotations


def sparse_bpw(M: int, K: int, nnz: int, col_bytes: int = 4, ptr_bytes: int = 4) -> float:
    """Extra bits/weight of the CSR part: FP16 value + column index per entry, plus row_ptr."""
    return (16 * nnz + 8 * col_bytes * nnz + 8 * ptr_bytes * (M + 1)) / (M * K)


def dense_bpw(bits: int, fmt: str, K: int, group: int = 16) -> float:
    """Bits/weight of the dense part: codes + FP16 (scale, zero) per group, or an FP16 LUT per row."""
    if fmt == "uniform":
        return bits + 2 * 16 / group
    if fmt == "lut":
        return bits + (1 << bits) * 16 / K
    raise ValueError(fmt)


def total_bpw(M: int, K: int, nnz: int, bits: int, fmt: str, group: int = 16, col_bytes: int = 4) -> float:
    return dense_bpw(bits, fmt, K, group) + sparse_bpw(M, K, nnz, col_bytes)
