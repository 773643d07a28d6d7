"""Unpermute and its gradient on the GPU vs the CPU oracle (needs an MI355X).

Integer-valued tokens and gradients with probabilities in {0.25, 0.5, 0.75, 1}
make every product and sum exact in fp32, so rounding once to the output type
gives the oracle's value bit for bit; random values are compared under the
normwise tolerance of the output type."""
import numpy as np
import pytest
import torch

import permute_grouped_gemm_amd as pgg
import synth
from gpu_util import to_torch

pytestmark = pytest.mark.gpu


def _inputs(batch, topk, H, dtype, seed, rit, exact):
    c = synth.make_case(batch, topk, 4 if topk <= 4 else topk, 1, 1, dtype, seed=seed, row_idx_type=rit)
    rng = np.random.default_rng(seed)
    if exact:
        perm = rng.integers(-2, 3, (c.M, H)).astype(np.float32)
        grad = rng.integers(-2, 3, (batch, H)).astype(np.float32)
        gm = rng.integers(-2, 3, (c.M, H)).astype(np.float32)
        probs = rng.choice(np.array([0.25, 0.5, 0.75, 1.0], np.float32), (batch, topk))
    else:
        perm = rng.standard_normal((c.M, H)).astype(np.float32)
        grad = rng.standard_normal((batch, H)).astype(np.float32)
        gm = rng.standard_normal((c.M, H)).astype(np.float32)
        probs = rng.random((batch, topk)).astype(np.float32)
    st = lambda a: synth.to_storage(a, dtype)
    return c, st(perm), st(probs), st(grad), st(gm)


def _dev(a, dtype):
    return to_torch(a, dtype).cuda()


def _host(t, dtype):
    t = t.cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype.itemsize == 2 else a.view(np.uint32)


# (5, 20, 264): more slots than one reduction batch of the register kernel;
# 4096 and 8200: rows at and past the register kernel's length limit.
SHAPES = [(100, 4, 300), (16, 8, 7168), (7, 1, 5), (513, 2, 1031), (5, 20, 264), (3, 2, 4096),
          (3, 2, 8200)]


def _draw_shapes(n, seed=20261208):
    # seeded (batch, topK, H) with H on both sides of the register kernel's limit
    rng = np.random.Generator(np.random.PCG64(seed))
    return [(int(rng.integers(1, 400)), int(rng.integers(1, 9)), int(rng.integers(1, 5000)))
            for _ in range(n)]


SHAPES += _draw_shapes(6)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rit", [0, 1])
def test_unpermute_exact(orc, shape, dtype, rit):
    batch, topk, H = shape
    c, perm, probs, grad, gm = _inputs(batch, topk, H, dtype, 70 + batch, rit, exact=True)
    eri = torch.from_numpy(c.eri).cuda()
    st = lambda a: synth.to_storage(np.asarray(a, dtype=np.float32), dtype)
    out = pgg.moe_unpermute(_dev(perm, dtype), eri, batch, topk, rit, _dev(probs, dtype))
    want = orc.moe_unpermute(perm, c.eri, rit, batch, topk, dtype, probs=probs)
    np.testing.assert_array_equal(_bits(_host(out, dtype)), _bits(st(want)))
    gat = pgg.moe_unpermute(_dev(perm, dtype), eri, batch, topk, rit)
    np.testing.assert_array_equal(_bits(_host(gat, dtype)),
                                  _bits(st(orc.moe_unpermute(perm, c.eri, rit, batch, topk, dtype))))
    pg, prg = pgg.moe_unpermute_grad(_dev(grad, dtype), eri, batch, topk, rit, _dev(perm, dtype),
                                     _dev(probs, dtype))
    wpg, wprg = orc.moe_unpermute_grad(grad, c.eri, rit, batch, topk, dtype, permuted=perm, probs=probs)
    np.testing.assert_array_equal(_bits(_host(pg, dtype)), _bits(st(wpg)))
    np.testing.assert_array_equal(_bits(_host(prg, dtype)), _bits(st(wprg)))
    sc, none = pgg.moe_unpermute_grad(_dev(gm, dtype), eri, batch, topk, rit)
    assert none is None
    wsc, _ = orc.moe_unpermute_grad(gm, c.eri, rit, batch, topk, dtype)
    np.testing.assert_array_equal(_bits(_host(sc, dtype)), _bits(st(wsc)))


# Results are stored in the input type (rounded once from fp32), so each
# element may differ from the exact value by the output type's rounding (half
# a unit in the last place) plus the fp32 summation error: bounded here by one
# unit in the last place, eps * |ref| with eps the type's spacing at 1, plus a
# tiny absolute term for elements near zero.
EPS = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}


def _close(got, ref, dtype, terms):
    bound = EPS[dtype] * np.abs(ref) + terms * 2.0 ** -24 * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (np.argwhere(bad)[:3], got[bad][:3], ref[bad][:3])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_unpermute_float(orc, dtype):
    batch, topk, H = 2048, 8, 7168
    c, perm, probs, grad, _ = _inputs(batch, topk, H, dtype, 90, 0, exact=False)
    eri = torch.from_numpy(c.eri).cuda()
    f = lambda a: synth.storage_to_f32(a, dtype).astype(np.float64)
    out = pgg.moe_unpermute(_dev(perm, dtype), eri, batch, topk, 0, _dev(probs, dtype))
    ref = orc.moe_unpermute(perm, c.eri, 0, batch, topk, dtype, probs=probs)
    _close(f(_host(out, dtype)), ref, dtype, 4 * topk)
    pg, prg = pgg.moe_unpermute_grad(_dev(grad, dtype), eri, batch, topk, 0, _dev(perm, dtype),
                                     _dev(probs, dtype))
    wpg, wprg = orc.moe_unpermute_grad(grad, c.eri, 0, batch, topk, dtype, permuted=perm, probs=probs)
    _close(f(_host(pg, dtype)), wpg, dtype, 4)
    _close(f(_host(prg, dtype)), wprg, dtype, 4 * H)


def test_unpermute_adjoint_on_gpu():
    batch, topk, H = 300, 4, 512
    c, perm, probs, grad, _ = _inputs(batch, topk, H, "f32", 91, 1, exact=False)
    eri = torch.from_numpy(c.eri).cuda()
    out = pgg.moe_unpermute(_dev(perm, "f32"), eri, batch, topk, 1, _dev(probs, "f32")).cpu().double()
    pg, prg = pgg.moe_unpermute_grad(_dev(grad, "f32"), eri, batch, topk, 1, _dev(perm, "f32"),
                                     _dev(probs, "f32"))
    a = float((out * torch.from_numpy(grad).double()).sum())
    b = float((prg.cpu().double() * torch.from_numpy(probs).double()).sum())
    d = float((pg.cpu().double() * torch.from_numpy(perm).double()).sum())
    scale = float(np.abs(grad).sum() * 4)
    assert abs(a - b) <= 1e-5 * scale and abs(a - d) <= 1e-5 * scale


def test_unpermute_index_errors():
    batch, topk, H = 10, 2, 8
    c, perm, probs, grad, _ = _inputs(batch, topk, H, "f32", 92, 0, exact=True)
    eri = c.eri.copy()
    eri[3] = eri[5]
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    pgg.moe_unpermute(_dev(perm, "f32"), torch.from_numpy(eri).cuda(), batch, topk, 0,
                      _dev(probs, "f32"), workspace=ws)
    code, detail = pgg.read_device_error(ws)
    assert code == pgg.DEV_INDEX_DUP
    eri[3] = 99
    pgg.moe_unpermute_grad(_dev(grad, "f32"), torch.from_numpy(eri).cuda(), batch, topk, 0,
                           _dev(perm, "f32"), _dev(probs, "f32"), workspace=ws)
    assert pgg.read_device_error(ws) == (pgg.DEV_INDEX_RANGE, 3)
    pgg.moe_unpermute(_dev(perm, "f32"), torch.from_numpy(c.eri).cuda(), batch, topk, 0,
                      _dev(probs, "f32"), workspace=ws)
    assert pgg.read_device_error(ws) == (pgg.DEV_OK, 0)
