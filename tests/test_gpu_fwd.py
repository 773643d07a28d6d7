"""The forward (Permute + GroupedMatmul) HIP path vs the CPU oracle, through
the C-ABI library (needs an MI355X).

Integer-valued inputs (|values| <= 2) keep every partial sum an integer below
2^24 (4 K <= 28672), so any summation order is exact and the HIP result must
equal the oracle bit for bit.  Random-valued inputs are compared with the
oracle's double result under the rules in parity.py (normwise 1e-5 for fp32 /
2e-3 for fp16 and bf16 inputs, and the elementwise a-priori bound over the K
terms of each element).
"""
import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import bits, run, to_torch, upload
from parity import check_close

pytestmark = pytest.mark.gpu


def upload_fwd(case, x):
    _, w, eri, gl = upload(case)
    return to_torch(x, case.dtype).to("cuda"), w, eri, gl


def run_fwd(case, x, tensors=None, workspace=None, out=None, check_error=True):
    xt, w, eri, gl = tensors if tensors is not None else upload_fwd(case, x)
    if workspace is None:
        workspace = torch.empty(pgg.fwd_workspace_size(xt, w, eri, gl, case.topk, case.row_idx_type),
                                dtype=torch.uint8, device="cuda")
    y = pgg.moe_fwd(xt, w, eri, gl, case.topk, case.row_idx_type, workspace=workspace, out=out)
    torch.cuda.synchronize()
    if check_error:
        assert pgg.read_device_error(workspace) == (pgg.DEV_OK, 0)
    return y.cpu().numpy()


def _check(orc, case, x, got, rows=None, what=""):
    ref, absdot = orc.case_fwd(case, x, rows=rows, want_abs=True)
    sel = got if rows is None else got[rows]
    return check_close(sel, ref, absdot, case.K, 1, case.dtype, what or case.name)


# ---------------------------------------------------------------- exact regime

FWD_SHAPES = [
    dict(batch=64, topk=2, G=4, K=256, N=128),                    # few rows per expert / fp32 tiles
    dict(batch=40, topk=8, G=16, K=7168, N=512, empty=(2, 5, 11)),  # long reduction, empty experts
    dict(batch=600, topk=4, G=5, K=600, N=300),                   # 256x256 tiles, K and N tails, W rows unaligned
    dict(batch=10, topk=3, G=4, K=178, N=286),                    # x rows unaligned
    dict(batch=700, topk=4, G=5, K=1000, N=2040),                 # 256x256 tiles, aligned, both tails
    dict(batch=4, topk=2, G=4, K=5, N=8),                         # one partial stage
    dict(batch=3, topk=1, G=1, K=16, N=4096),                     # one expert, 16 column tiles
    dict(batch=32, topk=8, G=16, K=520, N=264, routing="heavy", empty=(3,), heavy=5,
         heavy_rows=100),                                         # one expert with 4 m-tiles
    dict(batch=300, topk=2, G=2, K=64, N=256, row_idx_type=1),    # 256x256 tiles, scatter-form index
    dict(batch=20, topk=4, G=8, K=3000, N=520),                   # reduction split 5 ways, last one a tail
    dict(batch=20, topk=4, G=8, K=3001, N=520),                   # the same with unaligned x rows
]


@pytest.mark.parametrize("kw", FWD_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_forward_integer_inputs_bit_exact(orc, kw, dtype):
    case = synth.make_case(dtype=dtype, seed=900, integer=True, **kw)
    x = synth.forward_input(case, integer=True)
    print(f"[fwd] {kw} {dtype} plan {pgg.fwd_plan(*upload_fwd(case, x), case.topk, case.row_idx_type)}",
          flush=True)
    got = run_fwd(case, x)
    want = orc.case_fwd(case, x)
    assert 4 * case.K < 2 ** 24
    np.testing.assert_array_equal(bits(got), bits(want.astype(np.float32)))


@pytest.mark.parametrize("kw", FWD_SHAPES[:5] + FWD_SHAPES[7:])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_forward_float_parity(orc, kw, dtype):
    case = synth.make_case(dtype=dtype, seed=901, w_std=0.02, **kw)
    x = synth.forward_input(case)
    _check(orc, case, x, run_fwd(case, x))


def test_forward_ten_runs_bit_identical(orc):
    case = synth.make_case(700, 4, 5, 1000, 2040, "bf16", seed=902, w_std=0.02)
    x = synth.forward_input(case)
    t = upload_fwd(case, x)
    first = run_fwd(case, x, tensors=t)
    _check(orc, case, x, first)
    for _ in range(9):
        np.testing.assert_array_equal(bits(run_fwd(case, x, tensors=t)), bits(first))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_nan_in_empty_experts_never_read(orc, dtype):
    case = synth.make_case(50, 2, 6, 96, 320, dtype, seed=903, empty=(0, 3, 5), integer=True)
    x = synth.forward_input(case, integer=True)
    clean = run_fwd(case, x)
    w = case.weight.copy()
    w[[0, 3, 5]] = synth.to_storage(np.full((3, case.K, case.N), np.nan, np.float32), dtype)
    case.weight = w
    dirty = run_fwd(case, x)
    np.testing.assert_array_equal(bits(dirty), bits(clean))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_adjoint_with_gpu_backward(orc, dtype):
    # <y(x), d_y> == <x, d_x(d_y)> with both sides from the HIP library
    case = synth.make_case(200, 4, 8, 384, 512, dtype, seed=904, w_std=0.05)
    x = synth.forward_input(case)
    y = run_fwd(case, x).astype(np.float64)
    dx = run(case).astype(np.float64)
    dy = synth.storage_to_f32(case.grad_y, dtype).astype(np.float64)
    xf = synth.storage_to_f32(x, dtype).astype(np.float64)
    lhs = float(np.sum(y * dy))
    rhs = float(np.sum(xf * dx))
    scale = float(np.sum(np.abs(y * dy)) + np.sum(np.abs(xf * dx)))
    assert abs(lhs - rhs) <= 1e-5 * scale, (lhs, rhs, scale)


def test_forward_device_errors():
    base = dict(batch=32, topk=2, G=4, K=64, N=64, dtype="bf16", seed=905)
    c = synth.make_case(**base)
    x = synth.forward_input(c)
    t = upload_fwd(c, x)
    ws = torch.empty(pgg.fwd_workspace_size(*t, c.topk, 0), dtype=torch.uint8, device="cuda")
    eri = c.eri.copy()
    eri[7] = eri[3]
    bad = (t[0], t[1], torch.from_numpy(eri).cuda(), t[3])
    pgg.moe_fwd(*bad, c.topk, 0, workspace=ws)
    code, detail = pgg.read_device_error(ws)
    assert code == pgg.DEV_INDEX_DUP and detail == min(eri[3], eri[7])
    gl = c.group_list.copy()
    gl[0] += 1
    pgg.moe_fwd(t[0], t[1], t[2], torch.from_numpy(gl).cuda(), c.topk, 0, workspace=ws)
    assert pgg.read_device_error(ws) == (pgg.DEV_GROUP_SUM, c.M + 1)
    pgg.moe_fwd(*t, c.topk, 0, workspace=ws)
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)


def test_forward_kernel_time_hook_keeps_results(orc):
    case = synth.make_case(300, 4, 6, 512, 768, "f16", seed=906, w_std=0.02)
    x = synth.forward_input(case)
    t = upload_fwd(case, x)
    ws = torch.empty(pgg.fwd_workspace_size(*t, case.topk, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
    first = run_fwd(case, x, tensors=t, workspace=ws, out=out)
    ms = pgg.fwd_kernel_time(*t, case.topk, 0, repeats=3, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert ms > 0
    np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(first))
    _check(orc, case, x, first)


# ---------------------------------------------------------------- named workloads at full size

def _rows_sample(case, n=64, seed=0):
    """First and last rows, every expert's first and last row, and random rows."""
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(case.group_list)])
    edges = [off[g] for g in range(case.G) if case.group_list[g]] + \
            [off[g + 1] - 1 for g in range(case.G) if case.group_list[g]]
    return np.unique(np.concatenate([[0, case.M - 1], edges, rng.choice(case.M, n, replace=False)]))


def test_forward_decode_bf16_full(orc):
    case = synth.make_config("decode_bf16")
    x = synth.forward_input(case)
    _check(orc, case, x, run_fwd(case, x))


@pytest.mark.parametrize("name", ["mid_bf16", "large_f16", "large_f32_tail"])
def test_forward_workloads_sampled(orc, name):
    case = synth.make_config(name)
    x = synth.forward_input(case)
    got = run_fwd(case, x)
    rows = _rows_sample(case)
    _check(orc, case, x, got, rows=rows, what=name + " sampled rows")


@pytest.mark.parametrize("name", ["decode_bf16", "large_f16"])
def test_forward_integer_inputs_bit_exact_at_workload_shapes(orc, name):
    case = synth.make_config(name, integer=True)
    x = synth.forward_input(case, integer=True)
    got = run_fwd(case, x)
    rows = np.arange(case.M) if case.M <= 4096 else _rows_sample(case, seed=1)
    want = orc.case_fwd(case, x, rows=rows)
    np.testing.assert_array_equal(bits(got[rows]), bits(want.astype(np.float32)))
