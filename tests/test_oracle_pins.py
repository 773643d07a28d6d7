"""Pins of the CPU oracle against what the mathematics fixes (CPU only).

Each test pins the oracle to something other than itself: a library routine,
a literal brute-force evaluation, an identity between forward and backward,
an invariant, or the construction record of the input generator.  The
"planted mistake" tests at the end feed the oracle a plausibly wrong operand
and show that the corresponding pin fails.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import brute
from parity import check_close, gamma


def _args(c):
    return (c.grad_y, c.weight, c.eri, c.group_list, c.batch, c.topk, c.row_idx_type, c.dtype)


def _f64(c, x):
    return synth.storage_to_f32(x, c.dtype).astype(np.float64)


# ---------------------------------------------------------------- decoders

def test_half_decoder_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_decoder_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_generator_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    got = synth.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- brute force

TINY = [
    dict(batch=4, topk=2, G=3, K=5, N=7, seed=10),
    dict(batch=6, topk=3, G=4, K=3, N=9, seed=11, empty=(2,)),
    dict(batch=3, topk=1, G=2, K=8, N=4, seed=12),
    dict(batch=5, topk=3, G=4, K=4, N=5, seed=13, routing="heavy", empty=(0,), heavy=3, heavy_rows=6),
    dict(batch=1, topk=1, G=1, K=1, N=1, seed=14),
]


@pytest.mark.parametrize("kw", TINY)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_oracle_matches_literal_formula(orc, kw, dtype, row_idx_type):
    c = synth.make_case(dtype=dtype, row_idx_type=row_idx_type, **kw)
    lit = brute.dx_literal(_f64(c, c.grad_y), _f64(c, c.weight), c.eri, c.group_list,
                           c.batch, c.topk, c.row_idx_type)
    exact = orc.case_dx(c, mode=orc.EXACT)
    np.testing.assert_allclose(exact, lit, rtol=1e-13, atol=1e-13 * max(1.0, np.abs(lit).max()))
    slot, absdot = orc.case_dx(c, mode=orc.SLOT, want_abs=True)
    bound = (gamma(c.N + 1) + gamma(c.topk)) * absdot
    assert np.all(np.abs(slot.astype(np.float64) - lit) <= bound + 1e-300)


@pytest.mark.parametrize("kw", TINY)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_absdot_matches_literal_sum_of_magnitudes(orc, kw, dtype, row_idx_type):
    # the scale of every elementwise bound, term by term: sum |d_y| |W| over
    # the token's rows and the reduction, from all three oracle entries
    c = synth.make_case(dtype=dtype, row_idx_type=row_idx_type, **kw)
    lit = brute.absdot_literal(_f64(c, c.grad_y), _f64(c, c.weight), c.eri, c.group_list,
                               c.batch, c.topk, c.row_idx_type)
    assert np.all(lit >= 0)
    _, full = orc.case_dx(c, mode=orc.SLOT, want_abs=True)
    _, _, tok = orc.case_dx_tokens(c, np.arange(c.batch))
    cols = np.arange(c.K)[::-1].copy()
    _, _, col = orc.case_dx_cols(c, cols)
    for got in (full, tok, col[:, ::-1]):
        np.testing.assert_allclose(got, lit, rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("kw", TINY)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_column_subset_matches_literal_formula(orc, kw, dtype, row_idx_type):
    # every token at a subset of columns (repeats and any order allowed):
    # exact values against the literal formula; the float32 slot-order values
    # against the full slot-order evaluation bit for bit
    c = synth.make_case(dtype=dtype, row_idx_type=row_idx_type, **kw)
    lit = brute.dx_literal(_f64(c, c.grad_y), _f64(c, c.weight), c.eri, c.group_list,
                           c.batch, c.topk, c.row_idx_type)
    cols = np.array([c.K - 1, 0, c.K // 2, c.K - 1])
    d32, d64, ab = orc.case_dx_cols(c, cols)
    assert d32.shape == d64.shape == ab.shape == (c.batch, cols.size)
    np.testing.assert_allclose(d64, lit[:, cols], rtol=1e-13,
                               atol=1e-13 * max(1.0, np.abs(lit).max()))
    np.testing.assert_array_equal(d32.view(np.uint32), orc.case_dx(c, mode=orc.SLOT)[:, cols].view(np.uint32))


def test_column_subset_rejects_out_of_range_columns(orc):
    c = synth.make_case(4, 2, 3, 5, 7, "f32", seed=10)
    for bad in ([-1], [c.K]):
        with pytest.raises(orc.OracleError):
            orc.case_dx_cols(c, np.array(bad))


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_routing_single_expert_is_plain_matmul(orc, dtype):
    # topK = 1, G = 1, expanded row i is token i: d_x = d_y @ W[0]^T
    batch, K, N = 37, 29, 53
    expert = np.zeros((batch, 1), dtype=np.int64)
    c = synth.make_case(batch, 1, 1, K, N, dtype, seed=20, expert=expert)
    assert np.array_equal(c.eri, np.arange(batch))
    want = _f64(c, c.grad_y) @ _f64(c, c.weight)[0].T
    got = orc.case_dx(c, mode=orc.EXACT)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_identity_routing_many_experts_is_per_group_matmul(orc):
    # topK = 1, tokens sorted by expert so expanded order is identity
    G, K, N = 5, 11, 17
    counts = np.array([3, 0, 7, 1, 4])
    expert = np.repeat(np.arange(G), counts)[:, None]
    c = synth.make_case(int(counts.sum()), 1, G, K, N, "f32", seed=21, expert=expert)
    assert np.array_equal(c.eri, np.arange(c.batch))
    dy, W = _f64(c, c.grad_y), _f64(c, c.weight)
    want = np.zeros((c.batch, K))
    start = 0
    for g in range(G):
        want[start:start + counts[g]] = np.matmul(dy[start:start + counts[g]], W[g].T)
        start += counts[g]
    np.testing.assert_allclose(orc.case_dx(c, mode=orc.EXACT), want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- identities / invariants

@pytest.mark.parametrize("kw", TINY[:4] + [dict(batch=40, topk=4, G=6, K=16, N=24, seed=30)])
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_adjoint_identity(orc, kw, row_idx_type):
    # <d_x, x> == <d_y, GroupedMatmul(Permute(x), W)> for any x
    c = synth.make_case(dtype="f32", row_idx_type=row_idx_type, **kw)
    x = np.random.default_rng(kw["seed"]).standard_normal((c.batch, c.K))
    y = brute.forward_literal(x, _f64(c, c.weight), c.eri, c.group_list, c.topk, c.row_idx_type)
    lhs = float(np.sum(orc.case_dx(c, mode=orc.EXACT) * x))
    rhs = float(np.sum(_f64(c, c.grad_y) * y))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


def test_column_sum_invariant(orc):
    c = synth.make_case(50, 3, 5, 12, 20, "f32", seed=31)
    _, d64, _ = orc.dex(*_args(c), want64=True)
    dx = orc.case_dx(c, mode=orc.EXACT)
    np.testing.assert_allclose(dx.sum(axis=0), d64.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_colsum_matches_token_sums(orc):
    # the sum over expanded rows equals the sum over tokens of d_x (Step 2 regroups rows)
    c = synth.make_case(60, 4, 7, 20, 33, "bf16", seed=45, row_idx_type=1, empty=(3,))
    exact, absdot = orc.case_dx(c, mode=orc.EXACT, want_abs=True)
    cols = np.array([0, 7, 19, 7])
    s, a = orc.case_colsum(c, cols)
    np.testing.assert_allclose(s, exact.sum(0)[cols], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a, absdot.sum(0)[cols], rtol=1e-12)
    # and against a literal per-row evaluation in numpy
    dy, W = _f64(c, c.grad_y), _f64(c, c.weight)
    off = orc.offsets(c.group_list, c.M)
    lit = sum(dy[i] @ W[np.searchsorted(off, i, side="right") - 1, 19] for i in range(c.M))
    assert abs(s[2] - lit) <= 1e-12 * max(1.0, abs(lit))


@pytest.mark.parametrize("s", [-3, 5])
def test_power_of_two_scaling_is_bitwise(orc, s):
    c = synth.make_case(30, 2, 4, 9, 13, "f32", seed=32)
    base = orc.case_dx(c)
    c2 = synth.make_case(30, 2, 4, 9, 13, "f32", seed=32)
    c2.grad_y = (c.grad_y * np.float32(2.0 ** s)).astype(np.float32)
    np.testing.assert_array_equal(orc.case_dx(c2), base * np.float32(2.0 ** s))


def test_linearity(orc):
    # d_x(a + b) == d_x(a) + d_x(b); integer-valued a, b keep a + b exact in fp32
    a = synth.make_case(20, 2, 3, 6, 10, "f32", seed=33, integer=True)
    b = synth.make_case(20, 2, 3, 6, 10, "f32", seed=44, integer=True, expert=a.expert)
    b.weight = a.weight
    s = synth.make_case(20, 2, 3, 6, 10, "f32", seed=33, expert=a.expert)
    s.weight = a.weight
    s.grad_y = (a.grad_y + b.grad_y).astype(np.float32)
    np.testing.assert_array_equal(orc.case_dx(s, mode=orc.EXACT),
                                  orc.case_dx(a, mode=orc.EXACT) + orc.case_dx(b, mode=orc.EXACT))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_empty_experts_are_never_read(orc, dtype):
    c = synth.make_case(40, 2, 6, 10, 12, dtype, seed=34, empty=(1, 4))
    assert c.group_list[1] == 0 and c.group_list[4] == 0
    base = orc.case_dx(c)
    W = c.weight.copy()
    nan = synth.to_storage(np.full((c.K, c.N), np.nan, dtype=np.float32), dtype)
    W[1] = nan
    W[4] = nan
    c.weight = W
    got = orc.case_dx(c)
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got, base)


def test_inserting_an_empty_group_changes_nothing(orc):
    c = synth.make_case(25, 3, 4, 7, 9, "f32", seed=35)
    base = orc.case_dx(c)
    W = np.concatenate([c.weight[:2], np.full((1, c.K, c.N), np.nan, np.float32), c.weight[2:]])
    gl = np.concatenate([c.group_list[:2], [0], c.group_list[2:]])
    got = orc.moe_dx(c.grad_y, W, c.eri, gl, c.batch, c.topk, 0, "f32")
    np.testing.assert_array_equal(got, base)


@pytest.mark.parametrize("integer", [True, False])
def test_row_order_inside_a_group_does_not_matter(orc, integer):
    c = synth.make_case(30, 3, 4, 8, 10, "f32", seed=36, integer=integer)
    rng = np.random.default_rng(7)
    perm = np.arange(c.M)
    start = 0
    for cnt in c.group_list:
        perm[start:start + cnt] = start + rng.permutation(cnt)
        start += cnt
    # new expanded row r holds old row perm[r]
    shuffled = synth.make_case(30, 3, 4, 8, 10, "f32", seed=36, integer=integer)
    shuffled.grad_y = c.grad_y[perm]
    shuffled.eri = c.eri[perm]          # type 0: original position of the new row
    if integer:
        np.testing.assert_array_equal(orc.case_dx(shuffled), orc.case_dx(c))
    else:
        np.testing.assert_allclose(orc.case_dx(shuffled, mode=orc.EXACT),
                                   orc.case_dx(c, mode=orc.EXACT), rtol=1e-12, atol=1e-12)


def test_type0_and_type1_agree_bitwise(orc):
    a = synth.make_case(64, 4, 8, 16, 24, "bf16", seed=37, row_idx_type=0)
    b = synth.make_case(64, 4, 8, 16, 24, "bf16", seed=37, row_idx_type=1)
    assert not np.array_equal(a.eri, b.eri)
    np.testing.assert_array_equal(orc.case_dx(a), orc.case_dx(b))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_integer_inputs_are_exact_in_every_order(orc, dtype):
    c = synth.make_case(48, 4, 6, 20, 40, dtype, seed=38, integer=True)
    lit = brute.dx_literal(_f64(c, c.grad_y), _f64(c, c.weight), c.eri, c.group_list,
                           c.batch, c.topk, c.row_idx_type)
    for mode in (orc.SLOT, orc.ASCEND, orc.EXACT):
        np.testing.assert_array_equal(orc.case_dx(c, mode=mode).astype(np.float64), lit)


def test_index_normalisation_matches_construction(orc):
    for t in (0, 1):
        c = synth.make_case(100, 4, 7, 3, 3, "f32", seed=39, row_idx_type=t)
        ori, inv = orc.index(c.eri, t)
        np.testing.assert_array_equal(inv, c.rowpos.reshape(-1))
        np.testing.assert_array_equal(ori[inv], np.arange(c.M))
        # every (b, j) landed in a row of the expert it was routed to
        off = orc.offsets(c.group_list, c.M)
        g_of_row = np.searchsorted(off, np.arange(c.M), side="right") - 1
        np.testing.assert_array_equal(g_of_row[inv], c.expert.reshape(-1))


def test_token_subset_equals_full(orc):
    c = synth.make_case(40, 3, 5, 14, 22, "f16", seed=40, row_idx_type=1)
    full32 = orc.case_dx(c)
    full64, absdot = orc.case_dx(c, mode=orc.EXACT, want_abs=True)
    toks = np.array([39, 0, 17, 17, 5])
    d32, d64, ab = orc.case_dx_tokens(c, toks)
    np.testing.assert_array_equal(d32, full32[toks])
    np.testing.assert_array_equal(d64, full64[toks])
    np.testing.assert_array_equal(ab, absdot[toks])


def test_orders_agree_within_bound(orc):
    c = synth.make_config("tiny_f32")
    exact, absdot = orc.case_dx(c, mode=orc.EXACT, want_abs=True)
    for mode in (orc.SLOT, orc.ASCEND):
        check_close(orc.case_dx(c, mode=mode), exact, absdot, c.N, c.topk, "f32", f"mode{mode}")


# ---------------------------------------------------------------- constraints

def test_constraint_checks(orc):
    ok = dict(M=8, Ny=5, G=3, K=4, Nw=5, L=8, Gl=3, batch=4, topk=2, row_idx_type=0,
              dtype_y="f32", dtype_w="f32")
    assert orc.check(**ok) == orc.OK
    bad = [dict(Nw=6), dict(Gl=2), dict(L=7), dict(L=9), dict(M=9, L=9), dict(topk=0),
           dict(batch=0), dict(row_idx_type=2), dict(dtype_w="f16"), dict(dtype_y="f64", dtype_w="f64")]
    for b in bad:
        kw = dict(ok, **b)
        assert orc.check(**kw) == orc.ERR_SHAPE, b


def test_group_and_index_errors(orc):
    with pytest.raises(orc.OracleError) as e:
        orc.offsets(np.array([3, -1, 6]), 8)
    assert e.value.code == orc.ERR_GROUP_NEG
    with pytest.raises(orc.OracleError) as e:
        orc.offsets(np.array([3, 1, 3]), 8)
    assert e.value.code == orc.ERR_GROUP_SUM
    for t in (0, 1):
        with pytest.raises(orc.OracleError) as e:
            orc.index(np.array([0, 1, 8, 2]), t)
        assert e.value.code == orc.ERR_INDEX_RANGE
        with pytest.raises(orc.OracleError) as e:
            orc.index(np.array([0, 1, 1, 2]), t)
        assert e.value.code == orc.ERR_INDEX_DUP


# ---------------------------------------------------------------- planted mistakes

def test_planted_transposed_weight_fails_adjoint(orc):
    # a K<->N transpose of W (same shape when K == N) must break the adjoint pin
    c = synth.make_case(12, 2, 3, 6, 6, "f32", seed=41)
    x = np.random.default_rng(1).standard_normal((c.batch, c.K))
    y = brute.forward_literal(x, _f64(c, c.weight), c.eri, c.group_list, c.topk, 0)
    rhs = float(np.sum(_f64(c, c.grad_y) * y))
    wrong = orc.moe_dx(c.grad_y, np.ascontiguousarray(c.weight.transpose(0, 2, 1)), c.eri,
                       c.group_list, c.batch, c.topk, 0, "f32", mode=orc.EXACT)
    assert abs(float(np.sum(wrong * x)) - rhs) > 1e-6 * abs(rhs)


def test_planted_wrong_index_direction_fails_brute_force(orc):
    c = synth.make_case(8, 3, 4, 5, 6, "f32", seed=42, row_idx_type=0)
    lit = brute.dx_literal(_f64(c, c.grad_y), _f64(c, c.weight), c.eri, c.group_list,
                           c.batch, c.topk, 0)
    assert not np.array_equal(np.argsort(c.eri), c.eri)      # not an involution
    wrong = orc.moe_dx(*(_args(c)[:6]), 1, "f32", mode=orc.EXACT)
    assert np.abs(wrong - lit).max() > 1e-6 * np.abs(lit).max()


def test_planted_dropped_slot_fails_column_sum(orc):
    # dropping the last slot's contribution (topK read as topK-1 on a prefix of
    # tokens) breaks sum_b d_x[b,:] == sum_i d_expanded_x[i,:]
    c = synth.make_case(10, 3, 4, 5, 6, "f32", seed=43)
    _, d64, _ = orc.dex(*_args(c), want64=True)
    dx = orc.case_dx(c, mode=orc.EXACT)
    inv = c.rowpos.reshape(c.batch, c.topk)
    dropped = dx - d64[inv[:, -1]]
    assert np.abs(dropped.sum(0) - d64.sum(0)).max() > 1e-6
