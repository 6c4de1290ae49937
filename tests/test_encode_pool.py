"""The row-chunked oracle encoding used by the full-size GPU parity tests
equals the oracle's whole-matrix encoding, array for array."""

import numpy as np
import pytest

from encode_pool import encode_rows
from oracle import encode
from synth import WORKLOADS, make_weights, make_x, outlier_count


@pytest.mark.parametrize("name,M,K,chunk,nproc", [
    ("attn7b_u3", 40, 512, 16, 1),
    ("mlp7b_lut3", 24, 256, 8, 2),
    ("mlp70b_lut4", 33, 512, 10, 2),   # row-skewed law, two full outlier columns
    ("block7b_u3", 20, 352, 7, 1),
])
def test_chunked_encoding_equals_whole(name, M, K, chunk, nproc):
    wl = WORKLOADS[name]
    W, planted = make_weights(wl, 0, M, K)
    x = make_x(wl, 1, K, 0, M)
    sens = x[0].astype(np.float64) ** 2
    whole = encode.encode(W, wl.bits, wl.fmt, outlier_count(wl, M, K), wl.group or 16, sens=sens)
    parts = encode_rows(W, planted, wl.bits, wl.fmt, wl.group or 16, sens, chunk=chunk, nproc=nproc)
    for key in ("codes", "codes_packed", "mask", "scales", "zeros", "lut", "row_ptr", "col_idx", "values"):
        if key in whole:
            assert np.array_equal(np.asarray(whole[key]), np.asarray(parts[key])), key
            assert np.asarray(whole[key]).dtype == np.asarray(parts[key]).dtype, key


def test_chunked_encoding_catches_wrong_chunk_counts():
    """Chunk counts taken from the wrong rows (the planted mask shifted by one
    chunk) break the equality: the helper must count each chunk's own outliers."""
    wl = WORKLOADS["mlp7b_lut3"]
    W, planted = make_weights(wl, 0, 24, 256)
    x = make_x(wl, 1, 256, 0, 24)
    sens = x[0].astype(np.float64) ** 2
    whole = encode.encode(W, 3, "lut", outlier_count(wl, 24, 256), 16, sens=sens)
    shifted = np.roll(planted, 8, axis=0)
    assert [int(shifted[a:a + 8].sum()) for a in (0, 8, 16)] != [int(planted[a:a + 8].sum()) for a in (0, 8, 16)]
    wrong = encode_rows(W, shifted, 3, "lut", 16, sens, chunk=8, nproc=1)
    assert not np.array_equal(whole["row_ptr"], wrong["row_ptr"])
