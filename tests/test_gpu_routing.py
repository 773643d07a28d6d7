"""MoeInitRouting on the device vs the CPU oracle (needs an MI355X).

Routing is integer work: group_list, both index encodings and the permuted x
must equal the oracle's exactly."""
import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import to_torch

pytestmark = pytest.mark.gpu


def _route(expert, G, x=None, dtype="f32"):
    ids = torch.from_numpy(np.ascontiguousarray(expert, dtype=np.int64)).cuda()
    xt = to_torch(x, dtype).cuda() if x is not None else None
    ws = torch.empty(pgg.routing_workspace_size_desc(
        pgg.make_routing_desc(expert.shape[0], expert.shape[1], G,
                              0 if x is None else x.shape[1],
                              0 if x is None else pgg.DTYPE_CODE[xt.dtype])), dtype=torch.uint8,
        device="cuda")
    gl, eg, es, ex = pgg.moe_routing(ids, G, xt, workspace=ws)
    torch.cuda.synchronize()
    return gl.cpu().numpy(), eg.cpu().numpy(), es.cpu().numpy(), ex, ws


CASES = [
    dict(batch=1, topk=1, G=1, seed=1),
    dict(batch=16, topk=8, G=16, seed=2, empty=(1, 4, 9, 13)),          # decode-sized
    dict(batch=300, topk=4, G=7, seed=3),                               # two blocks
    dict(batch=2048, topk=8, G=16, seed=4, routing="zipf"),             # 16 blocks, skewed
    dict(batch=5000, topk=6, G=60, seed=5, routing="heavy", empty=(0, 59), heavy=7,
         heavy_rows=7500),                                              # duplicates inside tokens
    dict(batch=13824, topk=8, G=60, seed=6),                            # the large workload's routing
    dict(batch=700, topk=3, G=3000, seed=7),                            # many experts, most empty
    dict(batch=257, topk=4, G=8192, seed=8),                            # the expert limit
]


def _draw(n, seed=20261209):
    # seeded batch, topK and expert counts from one expert to a few thousand
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        G = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 4000))]))
        topk = int(rng.integers(1, min(G, 8) + 1))
        out.append(dict(batch=int(rng.integers(1, 6000)), topk=topk, G=G, seed=100 + i,
                        routing=("uniform", "zipf")[i % 2]))
    return out


CASES += _draw(8)


@pytest.mark.parametrize("kw", CASES)
def test_routing_tables_bit_exact(orc, kw):
    c = synth.make_case(K=1, N=1, **kw)
    print(f"[routing] {kw}", flush=True)
    gl, eg, es, _, ws = _route(c.expert, c.G)
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
    o_gl, o_t0, o_t1 = orc.moe_routing(c.expert, c.G)
    np.testing.assert_array_equal(gl, o_gl)
    np.testing.assert_array_equal(eg, o_t0)
    np.testing.assert_array_equal(es, o_t1)


# rows of one 4 KiB gather piece, several pieces with a short tail (bf16 7168),
# and rows that are not 16-byte multiples (byte copies), one of them three pieces
# long; the large batch takes 16 KiB pieces
@pytest.mark.parametrize("dtype,K", [("f32", 96), ("bf16", 7168), ("f16", 13), ("f16", 4099)])
def test_routing_expanded_x(orc, dtype, K):
    c = synth.make_case(300, 4, 9, K, 1, dtype, seed=20, empty=(2,))
    x = synth.forward_input(c)
    _, eg, _, ex, ws = _route(c.expert, c.G, x, dtype)
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
    want = np.ascontiguousarray(x[eg // c.topk])
    got = ex.cpu()
    if dtype == "bf16":
        got = got.view(torch.int16).numpy().view(np.uint16)
    else:
        got = got.numpy()
    np.testing.assert_array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("K", [3000, 9000])
def test_routing_expanded_x_large_batch(orc, K):
    # 2100 tokens take the 16 KiB pieces: rows of one piece and of two (16384 + 1616 bytes)
    c = synth.make_case(2100, 2, 8, K, 1, "bf16", seed=24)
    x = synth.forward_input(c)
    _, eg, _, ex, ws = _route(c.expert, c.G, x, "bf16")
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
    want = np.ascontiguousarray(x[eg // c.topk])
    got = ex.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_routing_feeds_the_operators(orc):
    # the device tables drive the fused backward to the same d_x as the generator's tables
    from gpu_util import run
    c = synth.make_case(64, 4, 8, 256, 128, "bf16", seed=21, integer=True)
    gl, eg, es, _, _ = _route(c.expert, c.G)
    np.testing.assert_array_equal(gl, c.group_list)
    np.testing.assert_array_equal(eg, c.eri)
    np.testing.assert_array_equal(run(c), orc.case_dx(c, mode=orc.SLOT))


def test_routing_range_error_and_recovery():
    c = synth.make_case(100, 4, 6, 1, 1, seed=22)
    bad = c.expert.copy()
    bad[30, 2] = 6
    bad[70, 0] = -1
    _, _, _, _, ws = _route(bad, c.G)
    assert pgg.read_device_error(ws) == (pgg.DEV_EXPERT_RANGE, 30 * 4 + 2)
    _, _, _, _, ws2 = _route(c.expert, c.G)
    assert pgg.read_device_error(ws2) == (pgg.DEV_OK, 0)


def test_routing_ten_runs_identical():
    c = synth.make_case(4000, 8, 60, 1, 1, seed=23)
    first = _route(c.expert, c.G)[:3]
    for _ in range(9):
        again = _route(c.expert, c.G)[:3]
        for a, b in zip(first, again):
            np.testing.assert_array_equal(a, b)
