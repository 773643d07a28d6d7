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


def test_readers_refuse_a_workspace_smaller_than_what_they_read():
    case = synth.make_case(16, 2, 4, 64, 32, "bf16", seed=2)
    gy, w, eri, gl = upload(case)
    ws = torch.empty(pgg.workspace_size(gy, w, eri, gl, case.batch, case.topk), dtype=torch.uint8,
                     device=gy.device)
    pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, workspace=ws)
    torch.cuda.synchronize()
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
    with pytest.raises(pgg.PggError) as e:
        pgg.read_device_error(ws[:32])
    assert e.value.status == pgg.ERR_INVALID_ARG
    with pytest.raises(pgg.PggError) as e:
        pgg.debug_tables(gy, w, eri, gl, case.batch, case.topk, 0, ws[:1024])
    assert e.value.status == pgg.ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(pgg.PggError) as e:
        pgg.debug_tiles(gy, w, eri, gl, case.batch, case.topk, 0, ws[:1024])
    assert e.value.status == pgg.ERR_WORKSPACE_TOO_SMALL
    inv, ori = pgg.debug_tables(gy, w, eri, gl, case.batch, case.topk, 0, ws)
    assert sorted(inv.tolist()) == list(range(case.M)) and sorted(ori.tolist()) == list(range(case.M))
