"""The oracle against hand-worked examples and the page's memory figures (CPU)."""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["handworked_2x2.json", "handworked_empty_dup.json"])
@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_handworked(orc, name, row_idx_type, dtype):
    fx = _load(name)
    dy = synth.to_storage(np.array(fx["grad_y"], dtype=np.float32), dtype)
    W = synth.to_storage(np.array(fx["weight"], dtype=np.float32), dtype)
    eri = np.array(fx["eri_type0" if row_idx_type == 0 else "eri_type1"], dtype=np.int64)
    gl = np.array(fx["group_list"], dtype=np.int64)
    args = (dy, W, eri, gl, fx["batch"], fx["topk"], row_idx_type, dtype)
    want = np.array(fx["d_x"], dtype=np.float64)
    for mode in (orc.SLOT, orc.ASCEND, orc.EXACT):
        got = orc.moe_dx(*args, mode=mode)
        np.testing.assert_array_equal(got.astype(np.float64), want)
    d32, _, _ = orc.dex(*args)
    np.testing.assert_array_equal(d32, np.array(fx["d_expanded_x"], dtype=np.float32))
    # the type-0 and type-1 encodings in the fixture describe the same routing
    ori, inv = orc.index(eri, row_idx_type)
    np.testing.assert_array_equal(ori, fx["eri_type0"])
    np.testing.assert_array_equal(inv, fx["eri_type1"])


def test_memory_figures():
    fx = _load("memory_figures.json")
    a = fx["d_expanded_x_fp16"]
    assert a["M"] * a["K"] * a["bytes_per_elem"] == a["exact"]
    assert abs(a["exact"] / 2 ** 30 - 1.5) < 0.03          # "about 1.5 GB"
    b = fx["d_expanded_x_fp32"]
    assert b["M"] * b["K"] * b["bytes_per_elem"] == b["exact"]
    assert abs(b["exact"] / 2 ** 30 - 3.0) < 0.05
    r = fx["ring_ascend"]
    assert r["parallNum"] * r["baseM"] * r["baseN"] * r["coreNum"] * r["bytes_per_elem"] == r["exact"]
    assert r["exact"] == 6 * 2 ** 20
    w = fx["d_weight_fp16"]
    assert w["G"] * w["K"] * w["N"] * w["bytes_per_elem"] == w["exact"]
    assert abs(w["exact"] / 2 ** 30 - 1.64) < 0.02           # page rounds to "about 1.7 GB"
