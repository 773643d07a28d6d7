"""Seeded random shapes across every producer family (needs an MI355X).

The plan picks the producer from the rows per expert (weight sweep, fp32
64- or 128-row tiles, 256 x 256 tiles; register-staged for rows that are not
16-byte aligned), so shapes drawn around those boundaries, with reduction
and column tails, exercise every kernel and its edges.  Integer-valued
inputs make every partial sum exact, so d_x must equal the oracle's
slot-ordered sum bit for bit.  The forward and the weight gradient are drawn
the same way, with aligned variants for their direct-to-LDS tiles.
"""
import numpy as np
import pytest

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import bits, run, upload

pytestmark = pytest.mark.gpu


def _draw(n, seed=20261203):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        dtype = ("f32", "f16", "bf16")[i % 3]
        G = int(rng.integers(1, 21))
        topk = int(rng.integers(1, min(G, 8) + 1))
        per = int(rng.choice([4, 12, 24, 30, 36, 48, 64, 96, 160, 300]))   # rows per expert
        batch = max(1, per * G // topk)
        K = int(rng.integers(1, 700))
        N = int(rng.choice([int(rng.integers(1, 300)), 64 * int(rng.integers(1, 5))]))
        out.append(dict(batch=batch, topk=topk, G=G, K=K, N=N, dtype=dtype))
    return out


# plus fp32 with many rows per expert (the direct-to-LDS 256 x 256 tile)
CASES = _draw(30) + [dict(batch=2400, topk=1, G=2, K=300, N=64, dtype="f32"),
                     dict(batch=1300, topk=2, G=2, K=260, N=70, dtype="f32")]


@pytest.mark.parametrize("kw", CASES, ids=[f"{c['dtype']}-b{c['batch']}k{c['topk']}G{c['G']}K{c['K']}N{c['N']}"
                                          for c in CASES])
def test_random_shape_bit_exact(orc, kw):
    case = synth.make_case(seed=7, integer=True, **kw)
    tensors = upload(case)
    plan = pgg.plan(*tensors, case.batch, case.topk, case.row_idx_type)
    print(f"[random] {kw} regime {plan['regime']} block {plan['block_m']}x{plan['block_n']}", flush=True)
    got = run(case, tensors=tensors)
    np.testing.assert_array_equal(bits(got), bits(orc.case_dx(case, mode=orc.SLOT)))


# every other drawn shape: all three types (the draw cycles them) and families
@pytest.mark.parametrize("kw", CASES[::2], ids=[f"{c['dtype']}-b{c['batch']}k{c['topk']}G{c['G']}K{c['K']}N{c['N']}"
                                               for c in CASES[::2]])
def test_random_shape_float_parity(orc, kw):
    # random values (weights N(0, 0.02)) against the oracle's exact sum, under
    # the normwise and elementwise tolerance rules
    from parity import check_close
    case = synth.make_case(seed=11, w_std=0.02, **kw)
    tensors = upload(case)
    print(f"[random float] {kw}", flush=True)
    got = run(case, tensors=tensors)
    exact, absdot = orc.case_dx(case, mode=orc.EXACT, want_abs=True)
    check_close(got, exact, absdot, case.N, case.topk, case.dtype, f"random {kw}")


# The forward and the weight gradient on shapes drawn the same way: their
# plans take the 32-row sweep up to 64 rows per expert, the 256 x 256 tiles
# above (direct-to-LDS when rows are 16-byte aligned) and 128 x 128 tiles for
# fp32.  Integer-valued x and weights keep every sum exact (|terms| <= 4, at
# most 700 of them for the forward and 300 * 8 rows per expert for d_weight).
def _aligned(cases):
    # K and N rounded up to multiples of 8: 16-byte rows, the direct-to-LDS paths
    return [dict(c, K=-(-c["K"] // 8) * 8, N=-(-c["N"] // 8) * 8) for c in cases]


FWD_CASES = _draw(18, seed=20261204) + _aligned(_draw(9, seed=20261206))
DW_CASES = _draw(18, seed=20261205) + _aligned(_draw(9, seed=20261207))


def _ids(cases):
    return [f"{c['dtype']}-b{c['batch']}k{c['topk']}G{c['G']}K{c['K']}N{c['N']}" for c in cases]


@pytest.mark.parametrize("kw", FWD_CASES, ids=_ids(FWD_CASES))
def test_random_shape_forward_bit_exact(orc, kw):
    from test_gpu_fwd import run_fwd, upload_fwd
    case = synth.make_case(seed=8, integer=True, **kw)
    x = synth.forward_input(case, integer=True)
    t = upload_fwd(case, x)
    print(f"[random fwd] {kw} plan {pgg.fwd_plan(*t, case.topk, case.row_idx_type)}", flush=True)
    got = run_fwd(case, x, tensors=t)
    np.testing.assert_array_equal(bits(got), bits(orc.case_fwd(case, x).astype(np.float32)))


@pytest.mark.parametrize("kw", DW_CASES, ids=_ids(DW_CASES))
def test_random_shape_dweight_bit_exact(orc, kw):
    from test_gpu_dw import run_dw, upload_dw
    case = synth.make_case(seed=9, integer=True, **kw)
    x = synth.forward_input(case, integer=True)
    t = upload_dw(case, x)
    print(f"[random dw] {kw} M {case.M}", flush=True)
    got = run_dw(case, x, tensors=t)
    assert 4 * int(np.max(case.group_list)) < 2 ** 24
    np.testing.assert_array_equal(bits(got), bits(orc.case_dw(case, x).astype(np.float32)))
