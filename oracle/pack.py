"""Canonical code bitstream -- test infrastructure only.

The pages ask for 3-4 bit codes stored densely ([SpQR] "Quantification d'un
modèle": wbits 3) but do not fix a bit order.  Reading: every row is one
contiguous little-endian bitstream; code j of a row occupies bits
[j*b, j*b + b) of that stream, least significant bit first, and row i starts
at byte i*K*b/8 (K*b is a multiple of 8).  For 4-bit codes this puts the
even-numbered code in the low nibble of each byte.
"""

from __future__ import annotations

import numpy as np


def pack_bitstream(codes: np.ndarray, bits: int) -> np.ndarray:
    """uint8 codes [M, K] (each < 2^bits) -> uint8 bytes [M, K*bits/8]."""
    codes = np.asarray(codes)
    M, K = codes.shape
    if (K * bits) % 8:
        raise ValueError("K*bits must be a multiple of 8")
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range")
    # bit t of code j goes to stream position j*bits + t
    bit_planes = (codes[:, :, None].astype(np.uint16) >> np.arange(bits)) & 1
    stream = bit_planes.reshape(M, K * bits).astype(np.uint8)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack_bitstream(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """uint8 bytes [M, K*bits/8] -> uint8 codes [M, K]; inverse of pack_bitstream."""
    packed = np.asarray(packed, dtype=np.uint8)
    M = packed.shape[0]
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, :K * bits]
    b = stream.reshape(M, K, bits).astype(np.uint16)
    return (b << np.arange(bits)).sum(axis=2).astype(np.uint8)
