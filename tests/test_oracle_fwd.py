"""Pins of the oracle's forward (Permute + GroupedMatmul), CPU only.

The forward of the MoeInitRoutingGroupedMatmulGrad design page (§数学定义和公式,
forward formulas): expanded_x = Permute(x), y[i, n] = sum_k expanded_x[i, k] *
W[g(i), k, n].  ``oracle.moe_fwd`` computes it with a per-expert float64
matmul; these tests pin it to things other than itself:

* hand-worked fixtures in ``tests/golden/`` (the same routing and weights as
  the backward fixtures, whose d_x they also satisfy the adjoint identity with);
* the literal per-row form in ``oracle/brute.py`` on tiny shapes;
* the adjoint identity <y(x), d_y> = <x, d_x(d_y)> against the C backward
  oracle, which its own pins tie to the page;
* a closed form: with W[g] = c_g * I, row i of y is c_g(i) times token
  p(i) // topK of x;
* planted mistakes (token = p % topK, a transposed weight, an off-by-one
  expert lookup) that each of these pins rejects.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(case, arr):
    return synth.storage_to_f32(arr, case.dtype).astype(np.float64)


@pytest.mark.parametrize("name", ["handworked_2x2.json", "handworked_empty_dup.json"])
@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_forward_handworked(orc, name, row_idx_type, dtype):
    with open(os.path.join(GOLDEN, name)) as f:
        fx = json.load(f)
    x = synth.to_storage(np.array(fx["x"], dtype=np.float32), dtype)
    W = synth.to_storage(np.array(fx["weight"], dtype=np.float32), dtype)
    eri = np.array(fx["eri_type0" if row_idx_type == 0 else "eri_type1"], dtype=np.int64)
    gl = np.array(fx["group_list"], dtype=np.int64)
    y = orc.moe_fwd(x, W, eri, gl, fx["batch"], fx["topk"], row_idx_type, dtype)
    np.testing.assert_array_equal(y, np.array(fx["y"], dtype=np.float64))
    # the fixture's forward and backward satisfy the adjoint identity exactly
    dy = np.array(fx["grad_y"], dtype=np.float64)
    dx = np.array(fx["d_x"], dtype=np.float64)
    assert float(np.sum(y * dy)) == float(np.sum(np.array(fx["x"], dtype=np.float64) * dx)) == fx["adjoint"]


TINY = [
    dict(batch=5, topk=2, G=3, K=4, N=6, seed=11),
    dict(batch=7, topk=3, G=4, K=9, N=5, seed=12, empty=(2,)),
    dict(batch=1, topk=1, G=1, K=3, N=2, seed=13),
    dict(batch=6, topk=3, G=5, K=2, N=7, seed=14, empty=(0, 4)),
    dict(batch=12, topk=3, G=4, K=5, N=3, seed=15, routing="heavy", empty=(1,), heavy=2, heavy_rows=15),
]


@pytest.mark.parametrize("kw", TINY)
@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_matches_literal(orc, kw, row_idx_type, dtype):
    c = synth.make_case(dtype=dtype, row_idx_type=row_idx_type, **kw)
    x = synth.forward_input(c)
    lit = brute.forward_literal(_f64(c, x), _f64(c, c.weight), c.eri, c.group_list, c.topk,
                                c.row_idx_type)
    y = orc.case_fwd(c, x)
    np.testing.assert_allclose(y, lit, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kw", TINY + [dict(batch=40, topk=4, G=6, K=16, N=24, seed=30),
                                       dict(batch=33, topk=2, G=5, K=40, N=13, seed=31, empty=(3,))])
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_forward_adjoint_with_backward_oracle(orc, kw, row_idx_type):
    # <GroupedMatmul(Permute(x), W), d_y> == <x, d_x(d_y)>, the backward from the C oracle
    c = synth.make_case(dtype="f32", row_idx_type=row_idx_type, **kw)
    x = synth.forward_input(c)
    y = orc.case_fwd(c, x)
    lhs = float(np.sum(y * _f64(c, c.grad_y)))
    rhs = float(np.sum(_f64(c, x) * orc.case_dx(c, mode=orc.EXACT)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_forward_scaled_identity_closed_form(orc, row_idx_type):
    # W[g] = c_g * I (K == N): y[i] = c_g(i) * x[p(i) // topK], exactly
    c = synth.make_case(9, 3, 4, 6, 6, "f32", seed=21, row_idx_type=row_idx_type, empty=(1,))
    scale = np.array([2.0, 0.0, -0.5, 3.0], dtype=np.float32)
    W = np.ascontiguousarray(scale[:, None, None] * np.eye(6, dtype=np.float32)[None])
    x = synth.forward_input(c, integer=True)
    y = orc.moe_fwd(x, W, c.eri, c.group_list, c.batch, c.topk, row_idx_type, "f32")
    expert_of = np.repeat(np.arange(4), c.group_list)
    pos = c.eri if row_idx_type == 0 else np.argsort(c.eri)
    want = scale[expert_of][:, None].astype(np.float64) * x[pos // c.topk].astype(np.float64)
    np.testing.assert_array_equal(y, want)


def test_forward_rows_subset_and_absdot(orc):
    c = synth.make_case(20, 3, 5, 11, 9, "f16", seed=22, empty=(2,))
    x = synth.forward_input(c)
    full, absfull = orc.case_fwd(c, x, want_abs=True)
    rows = np.array([0, 7, 59, 31, 7])
    part, abspart = orc.case_fwd(c, x, rows=rows, want_abs=True)
    np.testing.assert_array_equal(part, full[rows])
    np.testing.assert_array_equal(abspart, absfull[rows])
    assert np.all(absfull >= np.abs(full))


def test_forward_skips_empty_experts_nan(orc):
    c = synth.make_case(10, 2, 4, 5, 7, "f32", seed=23, empty=(0, 2))
    x = synth.forward_input(c)
    W = c.weight.copy()
    W[[0, 2]] = np.nan
    y = orc.moe_fwd(x, W, c.eri, c.group_list, c.batch, c.topk, 0, "f32")
    assert np.isfinite(y).all()
    np.testing.assert_array_equal(y, orc.case_fwd(c, x))


def test_forward_rejects_bad_inputs(orc):
    c = synth.make_case(4, 2, 3, 5, 6, "f32", seed=24)
    x = synth.forward_input(c)
    with pytest.raises(orc.OracleError):
        orc.moe_fwd(x[:, :4], c.weight, c.eri, c.group_list, c.batch, c.topk, 0, "f32")
    bad = c.group_list.copy()
    bad[0] += 1
    with pytest.raises(orc.OracleError) as e:
        orc.moe_fwd(x, c.weight, c.eri, bad, c.batch, c.topk, 0, "f32")
    assert e.value.code == orc.ERR_GROUP_SUM
    dup = c.eri.copy()
    dup[1] = dup[0]
    with pytest.raises(orc.OracleError) as e:
        orc.moe_fwd(x, c.weight, dup, c.group_list, c.batch, c.topk, 0, "f32")
    assert e.value.code == orc.ERR_INDEX_DUP


# ---------------------------------------------------------------- planted mistakes

def _fwd_variant(x, W, eri, group_list, topk, token_of, expert_side="right", transpose=False):
    """The forward with one step replaced (the mistakes the pins must catch)."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if transpose:
        W = W.transpose(0, 2, 1)
    M = eri.shape[0]
    off = np.concatenate([[0], np.cumsum(group_list)])
    g_of = np.searchsorted(off, np.arange(M), side=expert_side) - 1
    g_of = np.clip(g_of, 0, W.shape[0] - 1)
    return np.stack([x[token_of(eri[i], topk)] @ W[g_of[i]] for i in range(M)])


def test_planted_token_modulo_fails_golden():
    with open(os.path.join(GOLDEN, "handworked_2x2.json")) as f:
        fx = json.load(f)
    eri = np.array(fx["eri_type0"])
    wrong = _fwd_variant(fx["x"], fx["weight"], eri, np.array(fx["group_list"]), fx["topk"],
                         lambda p, t: p % t)
    right = _fwd_variant(fx["x"], fx["weight"], eri, np.array(fx["group_list"]), fx["topk"],
                         lambda p, t: p // t)
    np.testing.assert_array_equal(right, np.array(fx["y"], dtype=np.float64))
    assert not np.array_equal(wrong, np.array(fx["y"], dtype=np.float64))


def test_planted_expert_lookup_fails_golden():
    # side="left" puts a group's first row in the previous (here: empty) group
    with open(os.path.join(GOLDEN, "handworked_empty_dup.json")) as f:
        fx = json.load(f)
    W = np.nan_to_num(np.array(fx["weight"], dtype=np.float64), nan=0.0)
    eri = np.array(fx["eri_type0"])
    wrong = _fwd_variant(fx["x"], W, eri, np.array(fx["group_list"]), fx["topk"],
                         lambda p, t: p // t, expert_side="left")
    assert not np.array_equal(wrong, np.array(fx["y"], dtype=np.float64))


def test_planted_transposed_weight_fails_forward_adjoint(orc):
    c = synth.make_case(12, 2, 3, 6, 6, "f32", seed=41)
    x = synth.forward_input(c)
    rhs = float(np.sum(_f64(c, x) * orc.case_dx(c, mode=orc.EXACT)))
    wrong = _fwd_variant(_f64(c, x), _f64(c, c.weight), c.eri, c.group_list, c.topk,
                         lambda p, t: p // t, transpose=True)
    assert abs(float(np.sum(wrong * _f64(c, c.grad_y))) - rhs) > 1e-6 * abs(rhs)
    right = orc.case_fwd(c, x)
    assert abs(float(np.sum(right * _f64(c, c.grad_y))) - rhs) <= 1e-12 * abs(rhs)
