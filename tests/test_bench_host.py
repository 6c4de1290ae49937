"""bench.py's host helpers: stacked weight sets (--fuse) and the launch groups."""

import numpy as np
import pytest

import bench
from oracle import gemv
from synth import make_format_inputs, make_x


def part(name, M, K, seed_layer):
    f = make_format_inputs(name, seed_layer, M, K)
    f["row_ptr"], f["col_idx"], f["values"] = bench.csr_from_positions(f["M"], f["rows"], f["cols"], f["values"])
    return f


@pytest.mark.parametrize("name", ["block7b_u3", "mlp7b_lut3", "mlp7b_bpdq3", "mlp70b_lut4"])
def test_stacked_product_is_the_parts_products(name):
    """The oracle's y over stacked rows equals the parts' y one after another (fp64, exactly)."""
    K = 512
    parts = [part(name, M, K, 0) for M in (48, 16, 80)]  # the row count seeds each part
    f = bench.stack_rows(parts)
    assert f["M"] == 144 and f["row_ptr"][-1] == sum(p["row_ptr"][-1] for p in parts)
    x = make_x(name, 3, K, 0, 48)
    y, A = gemv.gemv_rows(f, x)
    ys = [gemv.gemv_rows(p, x) for p in parts]
    assert np.array_equal(y, np.concatenate([a for a, _ in ys], axis=1))
    assert np.array_equal(A, np.concatenate([b for _, b in ys], axis=1))


def test_stacking_rejects_mismatched_parts():
    a = part("block7b_u3", 16, 512, 0)
    b = part("block7b_u3", 16, 1024, 1)
    with pytest.raises(AssertionError):
        bench.stack_rows([a, b])


def test_launch_groups_cover_every_layer_once():
    units = bench.launch_units("block7b_u3", True)
    names = [n for _, members in units for _, n in members]
    assert names == [n for _, n in bench.workload_layers("block7b_u3")]
    assert [u for u, _ in units] == ["qkv", "o", "gate_up", "down"]
    assert bench.launch_units("mlp70b_lut4", True) == [("w", [(0, "w")])]
    assert len(bench.launch_units("block7b_u3", False)) == 7
