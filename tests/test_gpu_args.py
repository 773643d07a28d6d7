"""The binding refuses buffers on the wrong device or of the wrong shape
before any pointer reaches the library (needs an MI355X for GPU tensors)."""
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import upload

pytestmark = pytest.mark.gpu


def test_dx_out_and_workspace_must_be_on_the_inputs_gpu():
    case = synth.make_case(16, 2, 4, 64, 32, "bf16", seed=1)
    gy, w, eri, gl = upload(case)
    with pytest.raises(pgg.PggError):
        pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, out=torch.empty((case.batch, case.K)))
    with pytest.raises(pgg.PggError):
        pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(pgg.PggError):
        pgg.moe_dx(gy, w, eri.cpu(), gl, case.batch, case.topk)
    with pytest.raises(pgg.PggError):
        pgg.moe_dx_noalloc(gy, w, eri, gl, case.batch, case.topk, out=torch.empty((case.batch, case.K)))


def test_unpermute_arguments_checked_against_the_descriptor():
    batch, topk, H = 8, 2, 32
    dev = torch.device("cuda:0")
    perm = torch.zeros((batch * topk, H), dtype=torch.float16, device=dev)
    eri = torch.arange(batch * topk, dtype=torch.int64, device=dev)
    probs = torch.zeros((batch, topk), dtype=torch.float16, device=dev)
    with pytest.raises(pgg.PggError):    # too few rows
        pgg.moe_unpermute(perm[:-1], eri, batch, topk)
    with pytest.raises(pgg.PggError):    # probs of another dtype
        pgg.moe_unpermute(perm, eri, batch, topk, 0, probs.float())
    with pytest.raises(pgg.PggError):    # index of another type
        pgg.moe_unpermute(perm, eri.int(), batch, topk)
    with pytest.raises(pgg.PggError):    # gradient with probs needs permuted
        pgg.moe_unpermute_grad(torch.zeros((batch, H), dtype=torch.float16, device=dev), eri, batch, topk,
                               0, None, probs)
    out = pgg.moe_unpermute(perm, eri, batch, topk, 0, probs)
    torch.cuda.synchronize()
    assert out.shape == (batch, H)
