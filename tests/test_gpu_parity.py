"""HIP path vs the CPU oracle, through the C-ABI library (needs an MI355X).

Floating-point results are compared with the oracle's exact (double) d_x
under the rules in parity.py; integer-valued inputs make every summation
order exact, so there the HIP result must equal the oracle bit for bit; index
tables must match exactly; repeated calls must be bit-identical.
"""
import os

import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import bits, run, upload
from parity import check_close

pytestmark = pytest.mark.gpu


def _exact(orc, case):
    return orc.case_dx(case, mode=orc.EXACT, want_abs=True)


def _parity(orc, case, got=None):
    if got is None:
        got = run(case)
    exact, absdot = _exact(orc, case)
    return check_close(got, exact, absdot, case.N, case.topk, case.dtype, case.name)


# ---------------------------------------------------------------- small configs

def test_tiny_f32(orc):
    case = synth.make_config("tiny_f32")
    _parity(orc, case)


def test_tiny_f32_expert1_empty(orc):
    case = synth.make_config("tiny_f32", empty=(1,), seed=7)
    assert case.group_list[1] == 0
    _parity(orc, case)


@pytest.mark.parametrize("name,kw", synth.WHITEBOX, ids=[n for n, _ in synth.WHITEBOX])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_whitebox(orc, name, kw, dtype):
    kw = dict(kw)
    kw.setdefault("row_idx_type", 0)
    if name == "large_tokens" and dtype != "bf16":
        pytest.skip("large-token case runs once, in bf16")
    case = synth.make_case(dtype=dtype, seed=100, name=name, **kw)
    _parity(orc, case)


# ---------------------------------------------------------------- exact regime

EXACT_SHAPES = [
    dict(batch=64, topk=2, G=4, K=256, N=128),           # fp32 / several tiles
    dict(batch=40, topk=8, G=16, K=7168, N=512, empty=(2, 5, 11)),   # weight-streaming tiles
    dict(batch=600, topk=4, G=5, K=600, N=300),           # large tiles, row/col/reduction tails
    dict(batch=10, topk=3, G=4, K=178, N=286),            # unaligned rows (N*2 % 16 != 0)
    dict(batch=700, topk=4, G=5, K=1000, N=2040),         # large tiles, aligned rows, N % 64 != 0
    dict(batch=600, topk=4, G=5, K=600, N=286),           # large tiles, unaligned rows: register staged
    dict(batch=32, topk=8, G=16, K=512, N=256, routing="heavy", empty=(3,), heavy=0,
         heavy_rows=50),                                    # streaming, one m-tile per pass, 4 passes
    dict(batch=56, topk=8, G=16, K=520, N=264, routing="heavy", empty=(3,), heavy=5,
         heavy_rows=100),                                   # streaming, two m-tiles per pass, K/N tails
    dict(batch=4, topk=2, G=4, K=5, N=8),                  # streaming: one partial unit, one tiny stage
    dict(batch=4, topk=2, G=4, K=40, N=24),                # streaming: K not a multiple of 16
    dict(batch=3, topk=1, G=1, K=16, N=4096),              # streaming: one expert, one unit, 16 stages
]


@pytest.mark.parametrize("kw", EXACT_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_integer_inputs_bit_exact(orc, kw, dtype):
    case = synth.make_case(dtype=dtype, seed=200, integer=True, **kw)
    got = run(case)
    want = orc.case_dx(case, mode=orc.SLOT)
    np.testing.assert_array_equal(bits(got), bits(want))


def test_many_chunks_bit_exact(orc, monkeypatch):
    # a 1 MiB ring forces dozens of chunks: chunk-major order must still be exact
    monkeypatch.setenv("PGG_RING_MB", "1")
    monkeypatch.setenv("PGG_PANEL_COLS", "100000")   # one panel
    case = synth.make_case(300, 4, 6, 1024, 256, "bf16", seed=201, integer=True)
    gy, w, eri, gl = upload(case)
    plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, 0)
    assert plan["max_chunks"] >= 4, plan
    got = run(case, tensors=(gy, w, eri, gl))
    np.testing.assert_array_equal(bits(got), bits(orc.case_dx(case, mode=orc.SLOT)))


def test_many_chunks_stream_bit_exact(orc, monkeypatch):
    # few rows per expert (weight-sweep producer) split over many chunks,
    # with one expert above 32 rows so its m-tiles straddle chunks
    monkeypatch.setenv("PGG_RING_MB", "1")
    case = synth.make_case(56, 8, 16, 2048, 1024, "bf16", seed=203, integer=True, routing="heavy",
                           heavy=4, heavy_rows=60)
    gy, w, eri, gl = upload(case)
    plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, 0)
    assert plan["regime"] == 1 and plan["max_chunks"] >= 4, plan
    got = run(case, tensors=(gy, w, eri, gl))
    np.testing.assert_array_equal(bits(got), bits(orc.case_dx(case, mode=orc.SLOT)))


def test_many_chunks_float(orc, monkeypatch):
    monkeypatch.setenv("PGG_RING_MB", "2")
    case = synth.make_case(900, 4, 12, 768, 512, "f16", seed=202, w_std=0.02, name="chunked")
    _parity(orc, case)


# column panels x chunks: every panel runs the whole chunk sequence over its
# columns; ragged last panels (K tails) and both tiled producers
PANEL_CASES = [
    # (ring MiB, panel columns, case arguments)
    (1, 256, dict(batch=300, topk=4, G=6, K=1000, N=256, dtype="bf16")),    # 4 panels, last 232 wide
    (1, 512, dict(batch=300, topk=4, G=6, K=1000, N=256, dtype="f16")),     # 2 panels x chunks
    (1, 128, dict(batch=200, topk=4, G=5, K=600, N=264, dtype="f32")),      # fp32 tiles, one chunk per
                                                                             # panel, last panel 88 wide
    (1, 256, dict(batch=100, topk=3, G=4, K=700, N=286, dtype="bf16")),     # unaligned rows
    (4, 1024, dict(batch=600, topk=8, G=9, K=2000, N=512, dtype="bf16")),   # 7 chunks x 2 panels
    (32, 1024, dict(batch=600, topk=8, G=9, K=2000, N=512, dtype="bf16")),  # one chunk per panel
    # K not a multiple of 4: every consumer takes its 4-byte path
    (1, 256, dict(batch=300, topk=4, G=6, K=1001, N=256, dtype="bf16")),    # chunk consumer, 4 panels
    (1, 256, dict(batch=600, topk=8, G=9, K=1001, N=512, dtype="f16")),     # row consumer
    (1, 128, dict(batch=200, topk=4, G=5, K=601, N=264, dtype="f32")),      # token consumer, 5 panels
]


@pytest.mark.parametrize("ring_mb,cols,kw", PANEL_CASES)
def test_panels_bit_exact(orc, monkeypatch, ring_mb, cols, kw):
    monkeypatch.setenv("PGG_RING_MB", str(ring_mb))
    monkeypatch.setenv("PGG_PANEL_COLS", str(cols))
    case = synth.make_case(seed=204, integer=True, **kw)
    gy, w, eri, gl = upload(case)
    plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, 0)
    assert plan["n_panels"] == -(-case.K // plan["panel_cols"]) >= 2, plan
    got = run(case, tensors=(gy, w, eri, gl))
    np.testing.assert_array_equal(bits(got), bits(orc.case_dx(case, mode=orc.SLOT)))


def test_panels_float_and_repeatable(orc, monkeypatch):
    monkeypatch.setenv("PGG_RING_MB", "2")
    monkeypatch.setenv("PGG_PANEL_COLS", "256")
    case = synth.make_case(900, 4, 12, 1000, 512, "f16", seed=205, w_std=0.02, name="panels")
    gy, w, eri, gl = upload(case)
    plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, 0)
    assert plan["n_panels"] == 4 and plan["max_chunks"] >= 2, plan
    first = run(case, tensors=(gy, w, eri, gl))
    _parity(orc, case, first)
    for _ in range(3):
        np.testing.assert_array_equal(bits(run(case, tensors=(gy, w, eri, gl))), bits(first))


# ---------------------------------------------------------------- index tables

@pytest.mark.parametrize("row_idx_type", [0, 1])
@pytest.mark.parametrize("kw", [dict(batch=50, topk=3, G=7, K=64, N=64, empty=(4,)),
                                dict(batch=3000, topk=8, G=16, K=64, N=64)])
def test_index_tables_bit_exact(orc, row_idx_type, kw):
    case = synth.make_case(dtype="bf16", seed=300, row_idx_type=row_idx_type, **kw)
    gy, w, eri, gl = upload(case)
    ws = torch.empty(pgg.workspace_size(gy, w, eri, gl, case.batch, case.topk, row_idx_type),
                     dtype=torch.uint8, device="cuda")
    run(case, tensors=(gy, w, eri, gl), workspace=ws)
    inv, ori = pgg.debug_tables(gy, w, eri, gl, case.batch, case.topk, row_idx_type, ws)
    o_ori, o_inv = orc.index(case.eri, row_idx_type)
    np.testing.assert_array_equal(inv.numpy(), o_inv.astype(np.int32))
    np.testing.assert_array_equal(ori.numpy(), o_ori.astype(np.int32))
    tiles = pgg.debug_tiles(gy, w, eri, gl, case.batch, case.topk, row_idx_type, ws).numpy()
    bm = pgg.plan(gy, w, eri, gl, case.batch, case.topk, row_idx_type)["block_m"]
    off = orc.offsets(case.group_list, case.M)
    want = [(g, off[g] + s, min(bm, case.group_list[g] - s))
            for g in range(case.G) for s in range(0, int(case.group_list[g]), bm)]
    np.testing.assert_array_equal(tiles, np.array(want, dtype=np.int32).reshape(-1, 3))


# ---------------------------------------------------------------- invariants on the GPU

def test_type0_and_type1_bitwise(orc):
    a = synth.make_case(500, 8, 16, 512, 256, "bf16", seed=400, routing="zipf", row_idx_type=0)
    b = synth.make_case(500, 8, 16, 512, 256, "bf16", seed=400, routing="zipf", row_idx_type=1)
    ga, gb = run(a), run(b)
    np.testing.assert_array_equal(bits(ga), bits(gb))
    _parity(orc, a, ga)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_in_empty_experts_never_read(orc, dtype):
    case = synth.make_case(200, 4, 10, 384, 256, dtype, seed=401, empty=(0, 3, 9))
    base = run(case)
    W = case.weight.copy()
    nan = synth.to_storage(np.full((case.K, case.N), np.nan, np.float32), dtype)
    for g in (0, 3, 9):
        W[g] = nan
    case.weight = W
    got = run(case)
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(bits(got), bits(base))


def test_row_shuffle_inside_groups_integer(orc):
    case = synth.make_case(256, 4, 6, 320, 192, "f16", seed=402, integer=True)
    rng = np.random.default_rng(3)
    perm = np.arange(case.M)
    start = 0
    for cnt in case.group_list:
        perm[start:start + cnt] = start + rng.permutation(cnt)
        start += cnt
    shuffled = synth.make_case(256, 4, 6, 320, 192, "f16", seed=402, integer=True)
    shuffled.grad_y = case.grad_y[perm]
    shuffled.eri = case.eri[perm]
    np.testing.assert_array_equal(bits(run(shuffled)), bits(run(case)))


@pytest.mark.parametrize("kw", [
    dict(batch=16, topk=8, G=16, K=2048, N=1024, dtype="bf16", empty=(1, 5, 9)),   # weight sweep
    dict(batch=600, topk=8, G=9, K=2000, N=512, dtype="f16"),                     # large tiles
    dict(batch=200, topk=4, G=5, K=600, N=264, dtype="f32"),                       # fp32 tiles
    dict(batch=100, topk=3, G=4, K=700, N=286, dtype="bf16"),                      # unaligned rows
], ids=["sweep", "large", "f32", "unaligned"])
def test_power_of_two_scaling_bitwise(kw):
    # multiplying d_y by 4 multiplies every product and every partial sum by 4
    # exactly (random values, far from overflow and from the subnormals), so
    # d_x is 4 times the first result bit for bit, whatever order the sums take
    case = synth.make_case(seed=403, w_std=0.02, **kw)
    base = run(case)
    gy, w, eri, gl = upload(case)
    gy.mul_(4)
    got = run(case, tensors=(gy, w, eri, gl))
    np.testing.assert_array_equal(bits(got), bits(base * 4))


@pytest.mark.parametrize("which", ["tiny", "stream", "large", "chunked"])
def test_ten_runs_bit_identical(orc, which, monkeypatch):
    if which == "tiny":
        case = synth.make_config("tiny_f32")
    elif which == "stream":
        case = synth.make_case(16, 8, 16, 2048, 1024, "bf16", seed=500, empty=(1, 2, 3, 4))
    elif which == "large":
        case = synth.make_case(1024, 8, 8, 1024, 512, "f16", seed=501, w_std=0.02)
    else:
        monkeypatch.setenv("PGG_RING_MB", "2")
        case = synth.make_case(1024, 8, 60, 512, 256, "f32", seed=502, routing="heavy",
                               empty=tuple(range(0, 60, 5)), heavy=1, heavy_rows=2048)
    tensors = upload(case)
    first = run(case, tensors=tensors)
    for _ in range(9):
        np.testing.assert_array_equal(bits(run(case, tensors=tensors)), bits(first))


def test_concurrent_calls_on_two_streams():
    # calls share nothing but the inputs they are given: two problems (weight
    # sweep and large tiles) enqueued alternately on two streams, each with
    # its own workspace and output, give exactly their one-at-a-time results
    cases = [synth.make_case(16, 8, 16, 2048, 1024, "bf16", seed=503, empty=(2, 7)),
             synth.make_case(1024, 8, 8, 1024, 512, "f16", seed=504, w_std=0.02)]
    tensors = [upload(c) for c in cases]
    alone = [run(c, tensors=t) for c, t in zip(cases, tensors)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ws, outs = [], []
    for c, t in zip(cases, tensors):
        ws.append(torch.empty(pgg.workspace_size(*t, c.batch, c.topk, c.row_idx_type),
                              dtype=torch.uint8, device="cuda"))
        outs.append(torch.full((c.batch, c.K), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    for _ in range(3):
        for c, t, w, o, s in zip(cases, tensors, ws, outs, streams):
            pgg.moe_dx(*t, c.batch, c.topk, c.row_idx_type, out=o, workspace=w, stream=s)
    torch.cuda.synchronize()
    for c, w, o, want in zip(cases, ws, outs, alone):
        assert pgg.read_device_error(w) == (pgg.DEV_OK, 0)
        np.testing.assert_array_equal(bits(o.cpu().numpy()), bits(want))


# ---------------------------------------------------------------- device error word

def _err(case):
    gy, w, eri, gl = upload(case)
    ws = torch.empty(pgg.workspace_size(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type),
                     dtype=torch.uint8, device="cuda")
    pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type, workspace=ws)
    return pgg.read_device_error(ws)


@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_device_errors(row_idx_type):
    base = dict(batch=32, topk=2, G=4, K=64, N=64, dtype="bf16", seed=600, row_idx_type=row_idx_type)
    c = synth.make_case(**base)
    c.group_list = c.group_list.copy()
    c.group_list[1] -= 1
    c.group_list[2] += 1
    assert _err(c) == (pgg.DEV_OK, 0)          # still a valid split: no error
    c.group_list[0] = -1
    assert _err(c) == (pgg.DEV_GROUP_NEGATIVE, 0)
    c = synth.make_case(**base)
    c.group_list = c.group_list + np.array([0, 0, 0, 1])
    assert _err(c) == (pgg.DEV_GROUP_SUM, c.M + 1)
    c = synth.make_case(**base)
    c.eri = c.eri.copy()
    c.eri[5] = c.M
    assert _err(c) == (pgg.DEV_INDEX_RANGE, 5)
    c = synth.make_case(**base)
    c.eri = c.eri.copy()
    c.eri[7] = c.eri[3]
    code, detail = _err(c)
    assert code == pgg.DEV_INDEX_DUP and detail == min(c.eri[3], c.eri[7])
    # a valid call on the same workspace afterwards clears the word
    assert _err(synth.make_case(**base)) == (pgg.DEV_OK, 0)


# ---------------------------------------------------------------- named workloads at full size

def _sampled(orc, case, got, n=48, seed=0):
    rng = np.random.default_rng(seed)
    toks = np.unique(np.concatenate([[0, case.batch - 1], rng.choice(case.batch, n, replace=False)]))
    d32, d64, ab = orc.case_dx_tokens(case, toks)
    check_close(got[toks], d64, ab, case.N, case.topk, case.dtype, case.name + " sampled")
    cols = np.unique(np.concatenate([[0, case.K - 1], rng.choice(case.K, 6, replace=False)]))
    s, a = orc.case_colsum(case, cols)
    colsum = got[:, cols].astype(np.float64).sum(0)
    # the fp32 results of batch rows are summed in double; bound as for the elementwise check
    tol = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}[case.dtype]
    assert np.all(np.abs(colsum - s) <= tol * np.abs(s) + 8 * (case.N + case.topk) * 2.0 ** -24 * a), \
        (colsum, s)


def _edge_columns(case, n_extra=8, seed=0):
    """Both sides of every 256-column boundary (the large tiles' edges; panel
    edges and the fp32 path's 128-column tile edges at multiples of 256 are
    among them), the first and last column, and a few seeded others."""
    K = case.K
    edges = [c for m in range(256, K, 256) for c in (m - 1, m)]
    rng = np.random.default_rng(seed)
    extra = rng.choice(K, n_extra, replace=False)
    return np.array(sorted(set([0, K - 1] + edges + [int(c) for c in extra])), dtype=np.int64)


def _all_tokens_at_columns(orc, case, got, exact_bits):
    # every token, at ~64 columns that cross every tile and panel edge
    cols = _edge_columns(case)
    d32, d64, ab = orc.case_dx_cols(case, cols)
    if exact_bits:
        np.testing.assert_array_equal(bits(np.ascontiguousarray(got[:, cols])), bits(d32))
    else:
        check_close(got[:, cols], d64, ab, case.N, case.topk, case.dtype, case.name + " all tokens")
    return cols


def _ten_runs(case, first, tensors):
    # the plan these shapes get by default (column panels, chunk consumers)
    # must repeat bit for bit
    for _ in range(9):
        np.testing.assert_array_equal(bits(run(case, tensors=tensors)), bits(first))


def test_decode_bf16_full(orc):
    case = synth.make_config("decode_bf16")
    tensors = upload(case)
    first = run(case, tensors=tensors)
    _parity(orc, case, first)
    _ten_runs(case, first, tensors)


def test_mid_bf16_all_tokens(orc):
    case = synth.make_config("mid_bf16")
    tensors = upload(case)
    first = run(case, tensors=tensors)
    _sampled(orc, case, first)
    _all_tokens_at_columns(orc, case, first, exact_bits=False)
    _ten_runs(case, first, tensors)


def test_large_f16_all_tokens(orc):
    case = synth.make_config("large_f16")
    tensors = upload(case)
    first = run(case, tensors=tensors)
    _sampled(orc, case, first)
    _all_tokens_at_columns(orc, case, first, exact_bits=False)
    _ten_runs(case, first, tensors)


@pytest.mark.parametrize("name", ["large_f32", "large_f32_tail"])
def test_large_f32_all_tokens_and_deterministic(orc, name):
    case = synth.make_config(name)
    tensors = upload(case)
    first = run(case, tensors=tensors)
    _sampled(orc, case, first)
    _all_tokens_at_columns(orc, case, first, exact_bits=False)
    for _ in range(9):
        np.testing.assert_array_equal(bits(run(case, tensors=tensors)), bits(first))


# ---------------------------------------------------------------- preparation placement

@pytest.mark.parametrize("G,empty", [(64, (0, 63)), (80, (5,)), (256, (0, 100, 255)), (300, (7,))])
def test_stream_group_count_around_producer_preparation(orc, G, empty):
    # up to 256 groups the sweep producer prepares the indices itself (each
    # lane reading every 64th group); above, a preparation kernel runs first
    # -- both must give the oracle's result
    case = synth.make_case(40, 8, G, 512, 256, "bf16", seed=700, empty=empty, name=f"G{G}")
    gy, w, eri, gl = upload(case)
    assert pgg.plan(gy, w, eri, gl, case.batch, case.topk, 0)["regime"] == 1
    _parity(orc, case, run(case, tensors=(gy, w, eri, gl)))
    ws = torch.empty(pgg.workspace_size(gy, w, eri, gl, case.batch, case.topk, 0),
                     dtype=torch.uint8, device="cuda")
    run(case, tensors=(gy, w, eri, gl), workspace=ws)
    inv, ori = pgg.debug_tables(gy, w, eri, gl, case.batch, case.topk, 0, ws)
    o_ori, o_inv = orc.index(case.eri, 0)
    np.testing.assert_array_equal(inv.numpy(), o_inv.astype(np.int32))
    np.testing.assert_array_equal(ori.numpy(), o_ori.astype(np.int32))


# ---------------------------------------------------------------- benchmark hook

@pytest.mark.parametrize("which_case", ["stream", "chunked"])
def test_kernel_time_hook_keeps_results(orc, which_case, monkeypatch):
    if which_case == "stream":
        case = synth.make_case(16, 8, 16, 1024, 512, "bf16", seed=800, empty=(2, 7))
    else:
        monkeypatch.setenv("PGG_RING_MB", "1")
        case = synth.make_case(300, 4, 6, 1024, 256, "f16", seed=801, w_std=0.02)
    gy, w, eri, gl = upload(case)
    plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, 0)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
    out = torch.empty((case.batch, case.K), dtype=torch.float32, device="cuda")
    first = run(case, tensors=(gy, w, eri, gl), workspace=ws, out=out)
    for which in ("produce", "consume"):
        ms, launches = pgg.kernel_time(gy, w, eri, gl, case.batch, case.topk, 0, which=which,
                                       repeats=3, out=out, workspace=ws)
        assert ms > 0 and launches == plan["max_chunks"] * plan["n_panels"], (which, ms, launches)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(first))
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
    _parity(orc, case, first)


# ---------------------------------------------------------------- exact regime at the workloads' shapes

@pytest.mark.parametrize("name", ["decode_bf16", "mid_bf16", "large_f16", "large_f32",
                                  "large_f32_tail"])
def test_integer_inputs_bit_exact_at_workload_shapes(orc, name):
    # integer-valued inputs (|values| <= 2) at the named workloads' full
    # shapes: every partial sum is an integer below 2^24 (4 N topK <= 131072),
    # so any summation order is exact and the HIP result must equal the
    # oracle bit for bit -- on every token when the oracle does all of them
    # in seconds, else on a sample
    case = synth.make_config(name, integer=True)
    got = run(case)
    assert 4 * case.N * case.topk < 2 ** 24
    if case.M <= 4096:
        np.testing.assert_array_equal(bits(got), bits(orc.case_dx(case, mode=orc.SLOT)))
    else:
        # every token at ~64 columns across all tile and panel edges, and a
        # sample of whole token rows
        _all_tokens_at_columns(orc, case, got, exact_bits=True)
        rng = np.random.default_rng(2)
        toks = np.unique(np.concatenate([[0, case.batch - 1],
                                         rng.choice(case.batch, 16, replace=False)]))
        d32, _, _ = orc.case_dx_tokens(case, toks)
        np.testing.assert_array_equal(bits(got[toks]), bits(d32))
