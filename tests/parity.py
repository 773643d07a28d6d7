"""Tolerance rules shared by the parity tests.

The binding checks for floating-point results compare against the oracle's
exact (double) d_x:

* normwise: max|got - ref| / max|ref| <= tol, with tol = 1e-5 for fp32 inputs
  and 2e-3 for fp16 / bf16 inputs (fp32 accumulation in every case);
* elementwise: |got - ref| <= tol*|ref| + 4*(gamma(N+1) + gamma(topK)) * absdot,
  where gamma(n) = n*u / (1 - n*u), u = 2^-24, is the a-priori bound for an
  fp32 sum of n terms and absdot is the sum of |d_y|·|W| over the element's
  terms.  Near-zero elements make a plain relative error meaningless; this bound
  scales with the magnitude of the terms instead.
"""
import numpy as np

U32 = 2.0 ** -24
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def gamma(n: int) -> float:
    return n * U32 / (1.0 - n * U32)


def check_close(got, ref, absdot, N, topk, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    tol = TOL[dtype]
    err = np.abs(got - ref)
    refmax = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size and refmax > 0:
        normwise = float(np.max(err)) / refmax
        assert normwise <= tol, f"{what}: normwise rel err {normwise:.3e} > {tol:.1e}"
    bound = tol * np.abs(ref) + 4.0 * (gamma(N + 1) + gamma(topk)) * np.asarray(absdot, dtype=np.float64)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: elementwise bound violated at {tuple(idx)}: got {got[tuple(idx)]!r} "
                             f"ref {ref[tuple(idx)]!r} bound {bound[tuple(idx)]!r} ({int(bad.sum())} elements)")
    return float(np.max(err)) / refmax if refmax > 0 else 0.0
