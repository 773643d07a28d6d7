"""The fused backward captured into a HIP graph and replayed (needs an MI355X).

With its workspace and output passed in, a call enqueues kernels on the
caller's stream and nothing else: no allocation, no host copy, no memset (what
must start at zero is cleared by kernels). A caller can therefore capture it
into a HIP graph. The consumer's addition order is fixed, so every replay must
reproduce the eager result bit for bit. The replays are separated by eager
work and synchronisations, and each one runs on an output poisoned with NaN.
A replay after the inputs change in place must see the new inputs: doubling
d_y doubles d_x exactly on integer-valued inputs.
"""
import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import bits, upload

pytestmark = pytest.mark.gpu

# (id, environment, case) -- one per producer and consumer path
CASES = [
    # weight sweep with the index preparation inside its launch, token consumer
    ("sweep_prepared", {}, dict(batch=16, topk=8, G=16, K=2048, N=1024, dtype="bf16",
                                empty=(1, 5, 9))),
    # large tiles (direct-to-LDS stream), several chunks and column panels,
    # chunk consumer
    ("large_tiles_panels", {"PGG_RING_MB": "2", "PGG_PANEL_COLS": "256"},
     dict(batch=900, topk=4, G=12, K=1000, N=512, dtype="f16")),
    # large tiles, many chunks of one panel: row consumer
    ("large_tiles_rows", {"PGG_RING_MB": "1", "PGG_PANEL_COLS": "100000"},
     dict(batch=300, topk=4, G=6, K=1024, N=256, dtype="bf16")),
    # fp32 tiles (64 rows high here)
    ("f32_tiles", {}, dict(batch=200, topk=4, G=5, K=600, N=264, dtype="f32")),
    # fp32 weight sweep with the index preparation inside its launch
    ("f32_sweep_prepared", {}, dict(batch=16, topk=8, G=16, K=2048, N=1024, dtype="f32",
                                    empty=(2, 7))),
    # rows not 16-byte aligned: register-staged tiles
    ("unaligned_rows", {}, dict(batch=100, topk=3, G=4, K=700, N=286, dtype="bf16")),
]


def _replays_match(call, out, check, want, replays=3):
    """Capture call() once, then replay it with eager work in between; every
    replay must give `want` bit for bit."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    other = torch.arange(256 * 256, dtype=torch.float32, device="cuda").reshape(256, 256)
    for r in range(replays):
        out.fill_(float("nan"))
        float((other @ other).sum())        # eager work and a synchronisation
        g.replay()
        torch.cuda.synchronize()
        check()
        np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(want), err_msg=f"replay {r}")
    return g


@pytest.mark.parametrize("name,env,kw", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(monkeypatch, name, env, kw):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    case = synth.make_case(seed=950, integer=True, **kw)
    gy, w, eri, gl = upload(case)
    if env:
        plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type)
        assert plan["max_chunks"] >= 2, plan
    ws = torch.empty(pgg.workspace_size(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((case.batch, case.K), dtype=torch.float32, device="cuda")

    def call():
        pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type, out=out, workspace=ws)

    def check():
        assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)

    print(f"[graph] {name}: M={case.M} K={case.K} N={case.N} {case.dtype}", flush=True)
    call()
    torch.cuda.synchronize()
    check()
    eager = out.cpu().numpy()
    g = _replays_match(call, out, check, eager)
    # the graph reads the inputs at replay time
    gy.mul_(2)
    g.replay()
    torch.cuda.synchronize()
    check()
    np.testing.assert_array_equal(bits(out.cpu().numpy()), bits(eager * 2))


def test_graph_noalloc_replays_match_eager():
    # the allocation-free entry point is the one meant for callers that capture
    case = synth.make_case(600, 8, 9, 2000, 512, "bf16", seed=951, integer=True)
    gy, w, eri, gl = upload(case)
    out = torch.empty((case.batch, case.K), dtype=torch.float32, device="cuda")
    err = torch.full((2,), -7, dtype=torch.int64, device="cuda")

    def call():
        pgg.moe_dx_noalloc(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type, out=out,
                           device_error=err)

    def check():
        assert err.cpu().tolist() == [pgg.DEV_OK, 0]

    print(f"[graph] noalloc: M={case.M} K={case.K} N={case.N} {case.dtype}", flush=True)
    call()
    torch.cuda.synchronize()
    check()
    eager = out.cpu().numpy()
    _replays_match(call, out, lambda: (check(), err.fill_(-7)), eager)
