"""The allocation-free entry point (pgg_moe_dx_noalloc) against pgg_moe_dx,
through the C ABI (needs an MI355X).

The allocation-free call plans its ring to fit the library's fixed 64 MiB
scratch, so a problem whose regular ring is larger runs in more chunks there:
integer-valued inputs make every summation order exact, so both calls must
agree bit for bit; where both plans coincide, random inputs must agree bit for
bit too.  The scratch keeps the last call's contents, so a second, smaller
call right after the first must not see anything of it.
"""
import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import bits, run, upload

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _noalloc(case, tensors):
    gy, w, eri, gl = tensors
    out = torch.full((case.batch, case.K), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.full((2,), -7, dtype=torch.int64, device="cuda")
    pgg.moe_dx_noalloc(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type, out=out,
                       device_error=err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), err.cpu().numpy().tolist()


def test_noalloc_matches_moe_dx_on_two_calls_second_smaller():
    # call 1: a large-tile problem whose regular ring (157 MB, one chunk) does
    # not fit the scratch, so the allocation-free plan has more chunks
    big = synth.make_case(2400, 8, 12, 2048, 512, "bf16", seed=900, integer=True)
    tb = upload(big)
    plan = pgg.plan(*tb, big.batch, big.topk, big.row_idx_type)
    assert plan["ring_bytes"] > SCRATCH and plan["regime"] == 0, plan
    want = run(big, tensors=tb)
    got, err = _noalloc(big, tb)
    assert err == [pgg.DEV_OK, 0]
    np.testing.assert_array_equal(bits(got), bits(want))
    # call 2: smaller, random values, type-1 index; both plans are one chunk
    small = synth.make_case(300, 4, 6, 1000, 256, "f16", seed=901, w_std=0.02, row_idx_type=1)
    ts = upload(small)
    plan = pgg.plan(*ts, small.batch, small.topk, small.row_idx_type)
    assert plan["workspace_bytes"] < SCRATCH, plan
    want = run(small, tensors=ts)
    got, err = _noalloc(small, ts)
    assert err == [pgg.DEV_OK, 0]
    np.testing.assert_array_equal(bits(got), bits(want))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_weight_streaming_and_repeat(dtype):
    # decode-sized call (the weight sweep prepares the indices in its own
    # launch): equal to pgg_moe_dx bit for bit, and on a repeat
    case = synth.make_case(16, 8, 16, 2048, 1024, dtype, seed=902, empty=(1, 5, 9))
    t = upload(case)
    want = run(case, tensors=t)
    for _ in range(2):
        got, err = _noalloc(case, t)
        assert err == [pgg.DEV_OK, 0]
        np.testing.assert_array_equal(bits(got), bits(want))


def test_noalloc_reports_device_errors():
    case = synth.make_case(32, 2, 4, 64, 64, "bf16", seed=903)
    case.group_list = case.group_list + np.array([0, 0, 0, 1])
    _, err = _noalloc(case, upload(case))
    assert err == [pgg.DEV_GROUP_SUM, case.M + 1]
    # the next valid call on the same scratch reports no error
    ok = synth.make_case(32, 2, 4, 64, 64, "bf16", seed=903)
    t = upload(ok)
    got, err = _noalloc(ok, t)
    assert err == [pgg.DEV_OK, 0]
    np.testing.assert_array_equal(bits(got), bits(run(ok, tensors=t)))
