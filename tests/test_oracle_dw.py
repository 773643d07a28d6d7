"""Pins of the oracle's weight gradient (CPU only).

d_weight[g] = expanded_x_g^T · d_y_g (MoeInitRoutingGroupedMatmulGrad design
page, §1.2, the operator it leaves d_weight to).  ``oracle.moe_dw`` computes it
with one float64 matmul per expert; these tests pin it to:

* hand-worked values in both golden fixtures, whose <dW, W> equals the
  fixture's hand-worked <y, d_y> and <x, d_x>;
* the literal triple sum over (i, k, n) with an indicator [g(i) == g];
* the identity <dW(x, d_y), W> == <d_y, y(x, W)> against the pinned forward
  oracle and == <x, d_x(d_y, W)> against the C backward oracle;
* zeros for empty experts; expert subsets; rejections;
* planted mistakes (token p % topK, the expert's rows shifted by one, the
  operands swapped) that these pins catch.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(case, arr):
    return synth.storage_to_f32(arr, case.dtype).astype(np.float64)


@pytest.mark.parametrize("name", ["handworked_2x2.json", "handworked_empty_dup.json"])
@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dw_handworked(orc, name, row_idx_type, dtype):
    with open(os.path.join(GOLDEN, name)) as f:
        fx = json.load(f)
    x = synth.to_storage(np.array(fx["x"], dtype=np.float32), dtype)
    dy = synth.to_storage(np.array(fx["grad_y"], dtype=np.float32), dtype)
    eri = np.array(fx["eri_type0" if row_idx_type == 0 else "eri_type1"], dtype=np.int64)
    gl = np.array(fx["group_list"], dtype=np.int64)
    dw = orc.moe_dw(x, dy, eri, gl, fx["batch"], fx["topk"], row_idx_type, dtype)
    np.testing.assert_array_equal(dw, np.array(fx["d_weight"], dtype=np.float64))
    W = np.nan_to_num(np.array(fx["weight"], dtype=np.float64))
    assert float(np.sum(dw * W)) == fx["adjoint"]


def _literal(x, dy, eri, group_list, topk, row_idx_type, G):
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    M, N = dy.shape
    K = x.shape[1]
    g_of = np.repeat(np.arange(G), group_list)
    pos = np.asarray(eri) if row_idx_type == 0 else np.argsort(eri)
    out = np.zeros((G, K, N))
    for g in range(G):
        for i in range(M):
            ind = 1.0 if g_of[i] == g else 0.0
            for k in range(K):
                for n in range(N):
                    out[g, k, n] += ind * x[pos[i] // topk, k] * dy[i, n]
    return out


TINY = [
    dict(batch=5, topk=2, G=3, K=4, N=6, seed=51),
    dict(batch=7, topk=3, G=4, K=5, N=3, seed=52, empty=(2,)),
    dict(batch=1, topk=1, G=1, K=3, N=2, seed=53),
    dict(batch=9, topk=3, G=4, K=2, N=5, seed=54, routing="heavy", empty=(1,), heavy=3, heavy_rows=12),
]


@pytest.mark.parametrize("kw", TINY)
@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dw_matches_literal(orc, kw, row_idx_type, dtype):
    c = synth.make_case(dtype=dtype, row_idx_type=row_idx_type, **kw)
    x = synth.forward_input(c)
    lit = _literal(_f64(c, x), _f64(c, c.grad_y), c.eri, c.group_list, c.topk, row_idx_type, c.G)
    np.testing.assert_allclose(orc.case_dw(c, x), lit, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kw", TINY + [dict(batch=40, topk=4, G=6, K=16, N=24, seed=55),
                                       dict(batch=33, topk=2, G=5, K=40, N=13, seed=56, empty=(3,))])
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_dw_identities(orc, kw, row_idx_type):
    # <dW, W> == <d_y, y(x)> == <x, d_x(d_y)>, with y from the forward oracle and
    # d_x from the C backward oracle
    c = synth.make_case(dtype="f32", row_idx_type=row_idx_type, **kw)
    x = synth.forward_input(c)
    lhs = float(np.sum(orc.case_dw(c, x) * _f64(c, c.weight)))
    mid = float(np.sum(orc.case_fwd(c, x) * _f64(c, c.grad_y)))
    rhs = float(np.sum(_f64(c, x) * orc.case_dx(c, mode=orc.EXACT)))
    scale = max(1.0, abs(rhs))
    assert abs(lhs - mid) <= 1e-12 * scale and abs(lhs - rhs) <= 1e-12 * scale


def test_dw_empty_experts_zero_and_subset(orc):
    c = synth.make_case(12, 3, 6, 7, 9, "f16", seed=57, empty=(0, 4))
    x = synth.forward_input(c)
    full, absfull = orc.case_dw(c, x, want_abs=True)
    assert not full[[0, 4]].any()
    part, abspart = orc.case_dw(c, x, experts=[5, 0, 2], want_abs=True)
    np.testing.assert_array_equal(part, full[[5, 0, 2]])
    np.testing.assert_array_equal(abspart, absfull[[5, 0, 2]])
    assert np.all(absfull >= np.abs(full))


def test_dw_rejects_bad_inputs(orc):
    c = synth.make_case(4, 2, 3, 5, 6, "f32", seed=58)
    x = synth.forward_input(c)
    with pytest.raises(orc.OracleError):
        orc.moe_dw(x[:3], c.grad_y, c.eri, c.group_list, c.batch, c.topk, 0, "f32")
    bad = c.group_list.copy()
    bad[1] -= 1
    with pytest.raises(orc.OracleError) as e:
        orc.moe_dw(x, c.grad_y, c.eri, bad, c.batch, c.topk, 0, "f32")
    assert e.value.code == orc.ERR_GROUP_SUM


# ---------------------------------------------------------------- planted mistakes

def _dw_variant(x, dy, eri, group_list, topk, token_of=lambda p, t: p // t, shift=0, swap=False):
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    off = np.concatenate([[0], np.cumsum(group_list)])
    G = len(group_list)
    out = []
    for g in range(G):
        r = np.arange(off[g], off[g + 1])
        r = np.clip(r + shift, 0, len(eri) - 1) if r.size else r
        xg = x[token_of(np.asarray(eri)[r], topk)] if r.size else np.zeros((0, x.shape[1]))
        dyg = dy[r] if r.size else np.zeros((0, dy.shape[1]))
        out.append(dyg.T @ xg if swap else xg.T @ dyg)
    return out


def test_planted_mistakes_fail_golden():
    with open(os.path.join(GOLDEN, "handworked_2x2.json")) as f:
        fx = json.load(f)
    want = np.array(fx["d_weight"], dtype=np.float64)
    args = (fx["x"], fx["grad_y"], np.array(fx["eri_type0"]), np.array(fx["group_list"]), fx["topk"])
    np.testing.assert_array_equal(np.stack(_dw_variant(*args)), want)
    assert not np.array_equal(np.stack(_dw_variant(*args, token_of=lambda p, t: p % t)), want)
    assert not np.array_equal(np.stack(_dw_variant(*args, shift=1)), want)
    # swapped operands give the transpose: same shape here (K == N), different values
    assert not np.array_equal(np.stack(_dw_variant(*args, swap=True)), want)
