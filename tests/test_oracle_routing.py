"""Pins of the oracle's MoeInitRouting index outputs (CPU only).

``oracle.moe_routing`` places positions p = b*topK + j into expanded rows grouped
by expert, ascending p inside an expert, with plain loops.  It is pinned to the
hand-worked routing of the golden fixtures (group_list and both index
encodings were worked out by hand from the listed expert choices), to numpy's
stable argsort (the generator's independent construction), and to the
invariants of a permutation.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", ["handworked_2x2.json", "handworked_empty_dup.json"])
def test_routing_handworked(orc, name):
    with open(os.path.join(GOLDEN, name)) as f:
        fx = json.load(f)
    gl, t0, t1 = orc.moe_routing(np.array(fx["expert_ids"]), fx["G"])
    np.testing.assert_array_equal(gl, fx["group_list"])
    np.testing.assert_array_equal(t0, fx["eri_type0"])
    np.testing.assert_array_equal(t1, fx["eri_type1"])


@pytest.mark.parametrize("kw", [
    dict(batch=50, topk=4, G=7, seed=1),
    dict(batch=13, topk=3, G=9, seed=2, empty=(0, 8)),
    dict(batch=40, topk=8, G=16, seed=3, routing="zipf"),
    dict(batch=60, topk=4, G=6, seed=4, routing="heavy", empty=(2,), heavy=1, heavy_rows=100),
    dict(batch=1, topk=1, G=1, seed=5),
])
def test_routing_matches_stable_argsort(orc, kw):
    c = synth.make_case(K=1, N=1, **kw)
    gl, t0, t1 = orc.moe_routing(c.expert, c.G)
    np.testing.assert_array_equal(gl, c.group_list)
    np.testing.assert_array_equal(t0, np.argsort(c.expert.reshape(-1), kind="stable"))
    np.testing.assert_array_equal(t1, c.rowpos.reshape(-1))
    # a permutation and its inverse; rows grouped by expert; ascending p in a group
    np.testing.assert_array_equal(t1[t0], np.arange(c.M))
    ids = c.expert.reshape(-1)
    assert np.all(np.diff(ids[t0]) >= 0)
    same = np.diff(ids[t0]) == 0
    assert np.all(np.diff(t0)[same] > 0)


def test_routing_rejects_bad_ids(orc):
    with pytest.raises(orc.OracleError) as e:
        orc.moe_routing(np.array([[0, 3]]), 3)
    assert e.value.code == orc.ERR_INDEX_RANGE
    with pytest.raises(orc.OracleError):
        orc.moe_routing(np.array([[-1, 0]]), 3)


def test_planted_unstable_order_fails_golden(orc):
    # placing positions in descending p inside an expert breaks the hand-worked tables
    with open(os.path.join(GOLDEN, "handworked_empty_dup.json")) as f:
        fx = json.load(f)
    ids = np.array(fx["expert_ids"]).reshape(-1)
    wrong = np.argsort(ids * 1000 - np.arange(ids.size), kind="stable")
    assert not np.array_equal(wrong, fx["eri_type0"])
    gl, t0, _ = orc.moe_routing(ids, fx["G"])
    np.testing.assert_array_equal(t0, fx["eri_type0"])
