"""Pins of the oracle's unpermute and its gradient (CPU only).

MoeTokenUnpermute / MoeTokenUnpermuteGrad of the TileLang-Ascend operator
page (sections 4 and 5).  Pinned to hand-worked values (tests/golden, worked
on the first fixture's routing), to literal loops over (token, slot, h), and
to the adjoint identities of a bilinear map: <out(permuted, probs), grad> ==
<probs, probs_grad> == <permuted, perm_grad>, and for the gather,
<gather(permuted), grad> == <permuted, scatter(grad)>.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load():
    with open(os.path.join(GOLDEN, "handworked_2x2.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_unpermute_handworked(orc, row_idx_type, dtype):
    fx = _load()
    st = lambda a: synth.to_storage(np.array(a, dtype=np.float32), dtype)
    eri = np.array(fx["eri_type0" if row_idx_type == 0 else "eri_type1"])
    perm, probs, g = st(fx["y"]), st(fx["probs"]), st(fx["unpermute_grad_in"])
    out = orc.moe_unpermute(perm, eri, row_idx_type, fx["batch"], fx["topk"], dtype, probs=probs)
    np.testing.assert_array_equal(out, fx["unpermute_out"])
    gat = orc.moe_unpermute(perm, eri, row_idx_type, fx["batch"], fx["topk"], dtype)
    np.testing.assert_array_equal(gat, fx["unpermute_gather"])
    pg, prg = orc.moe_unpermute_grad(g, eri, row_idx_type, fx["batch"], fx["topk"], dtype,
                                     permuted=perm, probs=probs)
    np.testing.assert_array_equal(pg, fx["perm_grad"])
    np.testing.assert_array_equal(prg, fx["probs_grad"])
    assert float(np.sum(out * np.array(fx["unpermute_grad_in"]))) == \
        float(np.sum(np.array(fx["probs"]) * prg)) == 10.625


def _case(kw, dtype):
    c = synth.make_case(dtype=dtype, **kw)
    rng = np.random.default_rng(c.seed + 5)
    H = c.K
    perm = synth.to_storage(rng.standard_normal((c.M, H)).astype(np.float32), dtype)
    probs = synth.to_storage(rng.random((c.batch, c.topk)).astype(np.float32), dtype)
    g = synth.to_storage(rng.standard_normal((c.batch, H)).astype(np.float32), dtype)
    gm = synth.to_storage(rng.standard_normal((c.M, H)).astype(np.float32), dtype)
    return c, perm, probs, g, gm


KW = [dict(batch=6, topk=3, G=4, K=5, N=1, seed=61), dict(batch=9, topk=2, G=3, K=7, N=1, seed=62,
                                                            row_idx_type=1),
      dict(batch=1, topk=1, G=1, K=3, N=1, seed=63)]


@pytest.mark.parametrize("kw", KW)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpermute_matches_literal_loops(orc, kw, dtype):
    c, perm, probs, g, gm = _case(kw, dtype)
    f = lambda a: synth.storage_to_f32(a, dtype).astype(np.float64)
    P, PR, Gt = f(perm), f(probs), f(g)
    pos = c.eri if c.row_idx_type == 1 else np.argsort(c.eri)      # row of each position
    H = perm.shape[1]
    out = np.zeros((c.batch, H))
    pg = np.zeros((c.M, H))
    prg = np.zeros((c.batch, c.topk))
    for t in range(c.batch):
        for j in range(c.topk):
            r = pos[t * c.topk + j]
            for h in range(H):
                out[t, h] += PR[t, j] * P[r, h]
                pg[r, h] = Gt[t, h] * PR[t, j]
                prg[t, j] += Gt[t, h] * P[r, h]
    np.testing.assert_allclose(orc.moe_unpermute(perm, c.eri, c.row_idx_type, c.batch, c.topk, dtype,
                                                 probs=probs), out, rtol=1e-13, atol=1e-13)
    a, b = orc.moe_unpermute_grad(g, c.eri, c.row_idx_type, c.batch, c.topk, dtype, permuted=perm,
                                  probs=probs)
    np.testing.assert_allclose(a, pg, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(b, prg, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kw", KW + [dict(batch=40, topk=4, G=6, K=33, N=1, seed=64)])
def test_unpermute_adjoint_identities(orc, kw):
    c, perm, probs, g, gm = _case(kw, "f32")
    f = lambda a: np.asarray(a, dtype=np.float64)
    out = orc.moe_unpermute(perm, c.eri, c.row_idx_type, c.batch, c.topk, "f32", probs=probs)
    pg, prg = orc.moe_unpermute_grad(g, c.eri, c.row_idx_type, c.batch, c.topk, "f32", permuted=perm,
                                     probs=probs)
    a = float(np.sum(out * f(g)))
    b = float(np.sum(f(probs) * prg))
    d = float(np.sum(f(perm) * pg))
    scale = max(1.0, abs(a))
    assert abs(a - b) <= 1e-12 * scale and abs(a - d) <= 1e-12 * scale
    gat = orc.moe_unpermute(perm, c.eri, c.row_idx_type, c.batch, c.topk, "f32")
    sc, none = orc.moe_unpermute_grad(gm, c.eri, c.row_idx_type, c.batch, c.topk, "f32")
    assert none is None
    assert abs(float(np.sum(gat * f(gm))) - float(np.sum(f(perm) * sc))) <= 1e-12 * max(
        1.0, abs(float(np.sum(gat * f(gm)))))


def test_planted_transposed_slot_order_fails_golden(orc):
    # reading probs as [topK, batch] instead of [batch, topK] breaks the hand-worked output
    fx = _load()
    eri = np.array(fx["eri_type0"])
    probs_t = np.ascontiguousarray(np.array(fx["probs"], dtype=np.float32).T)
    out = orc.moe_unpermute(np.array(fx["y"], dtype=np.float32), eri, 0, 2, 2, "f32", probs=probs_t)
    assert not np.array_equal(out, fx["unpermute_out"])
