"""The weight gradient (expanded_x^T · d_y per expert) HIP path vs the CPU
oracle, through the C-ABI library (needs an MI355X).

Integer-valued inputs (|values| <= 2) keep every partial sum an integer below
2^24 (4 times an expert's row count), so any summation order is exact and the
HIP result must equal the oracle bit for bit.  Random-valued inputs are
compared with the oracle's double result under the rules in parity.py, with
the largest expert's row count as the reduction length.
"""
import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import bits, run, to_torch, upload
from parity import check_close
from test_gpu_fwd import FWD_SHAPES, run_fwd

pytestmark = pytest.mark.gpu


def upload_dw(case, x):
    gy, _, eri, gl = upload(case)
    return to_torch(x, case.dtype).to("cuda"), gy, eri, gl


def run_dw(case, x, tensors=None, workspace=None, out=None, experts=None, check_error=True):
    xt, gy, eri, gl = tensors if tensors is not None else upload_dw(case, x)
    if workspace is None:
        workspace = torch.empty(pgg.dw_workspace_size(xt, gy, eri, gl, case.topk, case.row_idx_type),
                                dtype=torch.uint8, device="cuda")
    dw = pgg.moe_dw(xt, gy, eri, gl, case.topk, case.row_idx_type, workspace=workspace, out=out)
    torch.cuda.synchronize()
    if check_error:
        assert pgg.read_device_error(workspace) == (pgg.DEV_OK, 0)
    if experts is not None:
        dw = dw[torch.as_tensor(np.asarray(experts), device=dw.device)]
    return dw.cpu().numpy()


def _check(orc, case, x, got, experts=None, what=""):
    ref, absdot = orc.case_dw(case, x, experts=experts, want_abs=True)
    rows = int(np.max(case.group_list)) if case.group_list.size else 1
    return check_close(got, ref, absdot, max(rows, 1), 1, case.dtype, what or case.name)


@pytest.mark.parametrize("kw", FWD_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dw_integer_inputs_bit_exact(orc, kw, dtype):
    case = synth.make_case(dtype=dtype, seed=950, integer=True, **kw)
    x = synth.forward_input(case, integer=True)
    print(f"[dw] {kw} {dtype}", flush=True)
    got = run_dw(case, x)
    want = orc.case_dw(case, x)
    assert 4 * int(np.max(case.group_list)) < 2 ** 24
    np.testing.assert_array_equal(bits(got), bits(want.astype(np.float32)))


@pytest.mark.parametrize("kw", FWD_SHAPES[:5] + FWD_SHAPES[7:])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dw_float_parity(orc, kw, dtype):
    case = synth.make_case(dtype=dtype, seed=951, **kw)
    x = synth.forward_input(case)
    _check(orc, case, x, run_dw(case, x))


def test_dw_ten_runs_bit_identical(orc):
    case = synth.make_case(700, 4, 5, 1000, 2040, "bf16", seed=952)
    x = synth.forward_input(case)
    t = upload_dw(case, x)
    first = run_dw(case, x, tensors=t)
    _check(orc, case, x, first)
    for _ in range(9):
        np.testing.assert_array_equal(bits(run_dw(case, x, tensors=t)), bits(first))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dw_empty_experts_are_zero(orc, dtype):
    case = synth.make_case(50, 2, 6, 96, 320, dtype, seed=953, empty=(0, 3, 5))
    x = synth.forward_input(case)
    t = upload_dw(case, x)
    out = torch.full((case.G, case.K, case.N), float("nan"), dtype=torch.float32, device="cuda")
    got = run_dw(case, x, tensors=t, out=out)
    assert np.all(bits(got[[0, 3, 5]]) == 0)          # +0.0 everywhere, NaN prefill overwritten
    _check(orc, case, x, got)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dw_identity_with_gpu_forward_and_backward(orc, dtype):
    # <dW, W> == <y, d_y> == <x, d_x>, every side from the HIP library
    case = synth.make_case(200, 4, 8, 384, 512, dtype, seed=954, w_std=0.05)
    x = synth.forward_input(case)
    dw = run_dw(case, x).astype(np.float64)
    y = run_fwd(case, x).astype(np.float64)
    dx = run(case).astype(np.float64)
    W = synth.storage_to_f32(case.weight, dtype).astype(np.float64)
    dy = synth.storage_to_f32(case.grad_y, dtype).astype(np.float64)
    xf = synth.storage_to_f32(x, dtype).astype(np.float64)
    a, b, c = float(np.sum(dw * W)), float(np.sum(y * dy)), float(np.sum(xf * dx))
    scale = float(np.sum(np.abs(dw * W)) + np.sum(np.abs(y * dy)))
    assert abs(a - b) <= 1e-5 * scale and abs(a - c) <= 1e-5 * scale, (a, b, c, scale)


def test_dw_device_errors():
    c = synth.make_case(32, 2, 4, 64, 64, "bf16", seed=955)
    x = synth.forward_input(c)
    t = upload_dw(c, x)
    ws = torch.empty(pgg.dw_workspace_size(*t, c.topk, 0), dtype=torch.uint8, device="cuda")
    eri = c.eri.copy()
    eri[5] = c.M
    pgg.moe_dw(t[0], t[1], torch.from_numpy(eri).cuda(), t[3], c.topk, 0, workspace=ws)
    assert pgg.read_device_error(ws) == (pgg.DEV_INDEX_RANGE, 5)
    pgg.moe_dw(*t, c.topk, 0, workspace=ws)
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
    with pytest.raises(pgg.PggError):
        pgg.moe_dw(t[0], t[1][:-2], t[2], t[3], c.topk, 0)


def test_dw_kernel_time_hook_keeps_results(orc):
    case = synth.make_case(300, 4, 6, 512, 768, "f16", seed=956)
    x = synth.forward_input(case)
    t = upload_dw(case, x)
    ws = torch.empty(pgg.dw_workspace_size(*t, case.topk, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.G, case.K, case.N), dtype=torch.float32, device="cuda")
    first = run_dw(case, x, tensors=t, workspace=ws, out=out)
    ms = pgg.dw_kernel_time(*t, case.topk, 0, repeats=3, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert ms > 0
    np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(first))
    _check(orc, case, x, first)


@pytest.mark.parametrize("name", ["decode_bf16", "mid_bf16", "large_f16"])
def test_dw_workloads_sampled_experts(orc, name):
    case = synth.make_config(name)
    x = synth.forward_input(case)
    nonempty = np.nonzero(case.group_list)[0]
    empty = np.nonzero(case.group_list == 0)[0]
    experts = sorted(set([int(nonempty[0]), int(nonempty[-1]), int(nonempty[len(nonempty) // 2])]
                         + [int(e) for e in empty[:1]]))
    got = run_dw(case, x, experts=experts)
    _check(orc, case, x, got, experts=experts, what=name + f" experts {experts}")


def test_dw_integer_bit_exact_at_decode_shape(orc):
    case = synth.make_config("decode_bf16", integer=True)
    x = synth.forward_input(case, integer=True)
    experts = list(range(case.G))
    got = run_dw(case, x, experts=experts)
    np.testing.assert_array_equal(bits(got), bits(orc.case_dw(case, x).astype(np.float32)))
