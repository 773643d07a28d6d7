"""CPU oracle for the fused MoE backward d_x (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the
``permute_grouped_gemm_amd`` package and its HIP library) never touches it,
and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, explicit loops, double
accumulation), which follows the formulas of the MoeInitRoutingGroupedMatmulGrad
design page, §数学定义和公式 (Step 1: d_expanded_x = d_y · Wᵀ per expert; Step 2:
scatter-add of expanded rows back to their token, batch row = original
position / topK).  ``brute.py`` evaluates the merged scalar formula of the same
section literally, with its indicator function, for tiny inputs.

``moe_fwd`` is the forward chain of the same section (MoeInitRouting =
Permute, then GroupedMatmul): expanded row i copies token p(i) / topK of x,
and every expert's rows are multiplied by that expert's weight slice, in
float64, with numpy's matmul as the per-expert product.  ``moe_dw`` is the
weight gradient the page leaves to a separate operator (§1.2):
expanded_x^T · d_y per expert, the same way.  ``moe_routing`` builds the
routing tables from router choices; ``moe_unpermute`` and
``moe_unpermute_grad`` are the TileLang-Ascend operator page's weighted
unpermute and its gradient.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (brute force, library matmul special cases, the
adjoint identity against an independent forward, invariants, hand-worked
fixtures in ``tests/golden/``); nothing is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, ERR_SHAPE, ERR_GROUP_NEG, ERR_GROUP_SUM, ERR_INDEX_RANGE, ERR_INDEX_DUP, ERR_ALLOC = range(7)
SLOT, ASCEND, EXACT = 0, 1, 2
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, no contraction of a*b+c)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared",
                               "-fPIC", "-pthread", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class _Problem(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("G", ctypes.c_int64),
                ("K", ctypes.c_int64), ("batch", ctypes.c_int64), ("topk", ctypes.c_int64),
                ("row_idx_type", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("grad_y", ctypes.c_void_p), ("weight", ctypes.c_void_p),
                ("eri", ctypes.c_void_p), ("group_list", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        PP = ctypes.POINTER(_Problem)
        L.orc_check.argtypes = [i64] * 9 + [i32] * 3
        L.orc_offsets.argtypes = [i64, vp, i64, vp]
        L.orc_index.argtypes = [i64, i32, vp, vp, vp]
        L.orc_decode.argtypes = [i32, vp, i64, vp]
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_dex.argtypes = [PP, vp, vp, vp, ctypes.c_int]
        L.orc_scatter.argtypes = [PP, vp, vp, vp, i32, vp, vp, vp]
        L.orc_dx_tokens.argtypes = [PP, vp, i64, vp, vp, vp, ctypes.c_int]
        L.orc_colsum.argtypes = [PP, vp, i64, vp, vp, ctypes.c_int]
        L.orc_dx_cols.argtypes = [PP, vp, i64, vp, vp, vp, ctypes.c_int]
        for f in ("orc_check", "orc_offsets", "orc_index", "orc_dex", "orc_scatter", "orc_dx_tokens",
                  "orc_colsum", "orc_dx_cols"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        super().__init__(f"oracle error {code} {what}")
        self.code = code


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _problem(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype):
    grad_y = np.ascontiguousarray(grad_y)
    weight = np.ascontiguousarray(weight)
    eri = np.ascontiguousarray(eri, dtype=np.int64)
    group_list = np.ascontiguousarray(group_list, dtype=np.int64)
    if grad_y.ndim != 2 or weight.ndim != 3 or eri.ndim != 1 or group_list.ndim != 1:
        raise OracleError(ERR_SHAPE, "rank")
    M, Ny = grad_y.shape
    G, K, Nw = weight.shape
    rc = lib().orc_check(M, Ny, G, K, Nw, eri.shape[0], group_list.shape[0], batch, topk,
                         row_idx_type, DTYPE_CODE[dtype], DTYPE_CODE[dtype])
    if rc:
        raise OracleError(rc, "shape")
    pr = _Problem(M, Ny, G, K, batch, topk, row_idx_type, DTYPE_CODE[dtype],
                  grad_y.ctypes.data, weight.ctypes.data, eri.ctypes.data, group_list.ctypes.data)
    keep = (grad_y, weight, eri, group_list)
    return pr, keep


def check(M, Ny, G, K, Nw, L, Gl, batch, topk, row_idx_type, dtype_y, dtype_w) -> int:
    return lib().orc_check(M, Ny, G, K, Nw, L, Gl, batch, topk, row_idx_type,
                           DTYPE_CODE.get(dtype_y, -1), DTYPE_CODE.get(dtype_w, -1))


def offsets(group_list: np.ndarray, M: int) -> np.ndarray:
    gl = np.ascontiguousarray(group_list, dtype=np.int64)
    off = np.zeros(gl.shape[0] + 1, dtype=np.int64)
    rc = lib().orc_offsets(gl.shape[0], gl.ctypes.data, M, off.ctypes.data)
    if rc:
        raise OracleError(rc, "group_list")
    return off


def index(eri: np.ndarray, row_idx_type: int):
    """(ori, inv): ori[i] original position of expanded row i, inv[p] expanded row of p."""
    eri = np.ascontiguousarray(eri, dtype=np.int64)
    M = eri.shape[0]
    ori = np.empty(M, dtype=np.int64)
    inv = np.empty(M, dtype=np.int64)
    rc = lib().orc_index(M, row_idx_type, eri.ctypes.data, ori.ctypes.data, inv.ctypes.data)
    if rc:
        raise OracleError(rc, "index")
    return ori, inv


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x)
    out = np.empty(x.size, dtype=np.float64)
    lib().orc_decode(DTYPE_CODE[dtype], x.ctypes.data, x.size, out.ctypes.data)
    return out.reshape(x.shape)


def dex(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype, *,
        want64=False, want_abs=False, nthreads=None):
    """Step 1: d_expanded_x rounded to float32 (and optionally the double values / |terms|)."""
    pr, keep = _problem(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype)
    d32 = np.empty((pr.M, pr.K), dtype=np.float32)
    d64 = np.empty((pr.M, pr.K), dtype=np.float64) if want64 else None
    a64 = np.empty((pr.M, pr.K), dtype=np.float64) if want_abs else None
    rc = lib().orc_dex(ctypes.byref(pr), _ptr(d32), _ptr(d64), _ptr(a64), nthreads or default_threads())
    if rc:
        raise OracleError(rc, "dex")
    return d32, d64, a64


def moe_dx(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype, *,
           mode=SLOT, want_abs=False, nthreads=None):
    """Full d_x [batch, K].  mode SLOT / ASCEND give float32, EXACT gives float64.

    With want_abs, also returns absdot[b,k] = sum over the token's terms of |d_y|·|W|."""
    d32, d64, a64 = dex(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype,
                        want64=(mode == EXACT), want_abs=want_abs, nthreads=nthreads)
    pr, keep = _problem(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype)
    dx32 = np.empty((batch, pr.K), dtype=np.float32) if mode != EXACT else None
    dx64 = np.empty((batch, pr.K), dtype=np.float64) if mode == EXACT else None
    absdot = np.empty((batch, pr.K), dtype=np.float64) if want_abs else None
    rc = lib().orc_scatter(ctypes.byref(pr), _ptr(d32), _ptr(d64), _ptr(a64), mode,
                           _ptr(dx32), _ptr(dx64), _ptr(absdot))
    if rc:
        raise OracleError(rc, "scatter")
    out = dx64 if mode == EXACT else dx32
    return (out, absdot) if want_abs else out


def moe_dx_tokens(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype, tokens, *,
                  nthreads=None):
    """d_x rows of the listed tokens: (slot-order float32, exact float64, absdot)."""
    pr, keep = _problem(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    dx32 = np.empty((n, pr.K), dtype=np.float32)
    dx64 = np.empty((n, pr.K), dtype=np.float64)
    absdot = np.empty((n, pr.K), dtype=np.float64)
    rc = lib().orc_dx_tokens(ctypes.byref(pr), tokens.ctypes.data, n, dx32.ctypes.data,
                             dx64.ctypes.data, absdot.ctypes.data, nthreads or default_threads())
    if rc:
        raise OracleError(rc, "tokens")
    return dx32, dx64, absdot


def moe_dx_cols(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype, cols, *,
                nthreads=None):
    """d_x of every token at the listed output columns: (slot-order float32,
    exact float64, absdot), each [batch, len(cols)].  Step 1 is evaluated
    only at those columns, so the cost is M * len(cols) * N multiply-adds."""
    pr, keep = _problem(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    n = cols.shape[0]
    dx32 = np.empty((batch, n), dtype=np.float32)
    dx64 = np.empty((batch, n), dtype=np.float64)
    absdot = np.empty((batch, n), dtype=np.float64)
    rc = lib().orc_dx_cols(ctypes.byref(pr), cols.ctypes.data, n, dx32.ctypes.data,
                           dx64.ctypes.data, absdot.ctypes.data, nthreads or default_threads())
    if rc:
        raise OracleError(rc, "cols")
    return dx32, dx64, absdot


def colsum(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype, cols, *,
           nthreads=None):
    """(sum over all tokens of d_x[:, k], matching sum of |terms|) for k in cols, in double."""
    pr, keep = _problem(grad_y, weight, eri, group_list, batch, topk, row_idx_type, dtype)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    s = np.empty(cols.shape[0], dtype=np.float64)
    a = np.empty(cols.shape[0], dtype=np.float64)
    rc = lib().orc_colsum(ctypes.byref(pr), cols.ctypes.data, cols.shape[0], s.ctypes.data,
                          a.ctypes.data, nthreads or default_threads())
    if rc:
        raise OracleError(rc, "colsum")
    return s, a


def moe_fwd(x, weight, eri, group_list, batch, topk, row_idx_type, dtype, *, rows=None,
            want_abs=False):
    """Forward y[i, n] = sum_k x[p(i) // topK, k] * W[g(i), k, n] in float64.

    MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式, forward
    formulas: expanded_x = Permute(x) (row i copies token p(i) // topK, with
    p(i) the original position of expanded row i), then the grouped matmul of
    §1.1 step 2, each expert's expanded rows times its weight slice W[g]
    ([K, N]).  x is [batch, K], weight [G, K, N], both in the storage type
    ``dtype``; eri, group_list and row_idx_type as for moe_dx.  ``rows``
    (optional) selects expanded rows; the result has one row per entry.  With
    want_abs, also returns absdot[i, n] = sum_k |x|·|W| over the same terms.
    Only the weight slices of experts that own a selected row are decoded.
    """
    x = np.ascontiguousarray(x)
    weight = np.ascontiguousarray(weight)
    if x.ndim != 2 or weight.ndim != 3:
        raise OracleError(ERR_SHAPE, "rank")
    G, K, N = weight.shape
    M = batch * topk
    if x.shape != (batch, K) or np.shape(eri) != (M,) or np.shape(group_list) != (G,):
        raise OracleError(ERR_SHAPE, "shape")
    off = offsets(group_list, M)
    ori, _ = index(eri, row_idx_type)
    sel = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if sel.size and (sel.min() < 0 or sel.max() >= M):
        raise OracleError(ERR_INDEX_RANGE, "rows")
    # g(i): the expert whose row range [off[g], off[g+1]) holds i
    g_of = np.searchsorted(off, sel, side="right") - 1
    y = np.zeros((sel.size, N), dtype=np.float64)
    absdot = np.zeros((sel.size, N), dtype=np.float64) if want_abs else None
    for g in np.unique(g_of):
        at = np.nonzero(g_of == g)[0]
        tokens = ori[sel[at]] // topk
        xg = decode(x[tokens], dtype)
        wg = decode(weight[g], dtype)
        y[at] = xg @ wg
        if want_abs:
            absdot[at] = np.abs(xg) @ np.abs(wg)
    return (y, absdot) if want_abs else y


def moe_dw(x, grad_y, eri, group_list, batch, topk, row_idx_type, dtype, *, experts=None,
           want_abs=False):
    """Weight gradient dW[g, k, n] = sum over expert g's expanded rows i of
    x[p(i) // topK, k] * grad_y[i, n], in float64.

    MoeInitRoutingGroupedMatmulGrad design page, §1.2 (why d_weight is left
    to a separate operator): d_weight [G, K, N] = expanded_x^T @ d_y per
    expert, with expanded_x = Permute(x) as in the forward formulas of
    §数学定义和公式.  x is [batch, K], grad_y [M, N], in the storage type
    ``dtype``.  An expert with no rows gets zeros.  ``experts`` (optional)
    selects experts; the result has one [K, N] slice per entry.  With
    want_abs, also returns the sums of |x|·|grad_y| over the same terms.
    """
    x = np.ascontiguousarray(x)
    grad_y = np.ascontiguousarray(grad_y)
    if x.ndim != 2 or grad_y.ndim != 2:
        raise OracleError(ERR_SHAPE, "rank")
    M = batch * topk
    G = int(np.shape(group_list)[0])
    K, N = x.shape[1], grad_y.shape[1]
    if x.shape[0] != batch or grad_y.shape[0] != M or np.shape(eri) != (M,):
        raise OracleError(ERR_SHAPE, "shape")
    off = offsets(group_list, M)
    ori, _ = index(eri, row_idx_type)
    sel = np.arange(G) if experts is None else np.asarray(experts, dtype=np.int64)
    dw = np.zeros((sel.size, K, N), dtype=np.float64)
    absdot = np.zeros((sel.size, K, N), dtype=np.float64) if want_abs else None
    for at, g in enumerate(sel):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        xg = decode(x[ori[r0:r1] // topk], dtype)        # expanded_x rows of expert g
        dyg = decode(grad_y[r0:r1], dtype)
        dw[at] = xg.T @ dyg
        if want_abs:
            absdot[at] = np.abs(xg).T @ np.abs(dyg)
    return (dw, absdot) if want_abs else dw


def case_dw(case, x, **kw):
    """moe_dw on a ``synth.Case`` (its grad_y and routing) and activations x."""
    return moe_dw(x, case.grad_y, case.eri, case.group_list, case.batch, case.topk,
                  case.row_idx_type, case.dtype, **kw)


def moe_routing(expert_ids, G):
    """MoeInitRouting's index outputs from the router's choices (CPU, plain loops).

    MoeInitRoutingGroupedMatmulGrad design page, §1.1 step 1 (MoeInitRouting,
    semantically a permute: tokens are grouped by expert) with the original
    position p = b * topK + j of §数学定义和公式.  Expanded rows are grouped by
    expert in expert order, and inside an expert they keep ascending p (the
    page fixes no order there; this stable order is the reading taken).
    Returns (group_list int64 [G] counts, eri_type0 int64 [M]: original
    position of each expanded row, eri_type1 int64 [M]: expanded row of each
    position).  Raises OracleError(ERR_INDEX_RANGE) for an id outside [0, G).
    """
    ids = np.asarray(expert_ids, dtype=np.int64).reshape(-1)
    M = ids.size
    counts = [0] * G
    for p in range(M):
        e = int(ids[p])
        if e < 0 or e >= G:
            raise OracleError(ERR_INDEX_RANGE, f"expert id {e} at position {p}")
        counts[e] += 1
    start = [0] * G
    for g in range(1, G):
        start[g] = start[g - 1] + counts[g - 1]
    nxt = list(start)
    type0 = np.empty(M, dtype=np.int64)
    type1 = np.empty(M, dtype=np.int64)
    for p in range(M):                       # ascending p: a stable placement
        e = int(ids[p])
        row = nxt[e]
        nxt[e] += 1
        type0[row] = p
        type1[p] = row
    return np.array(counts, dtype=np.int64), type0, type1


def _rows_of_positions(eri, row_idx_type):
    """inv[p]: the expanded row of original position p (validated permutation)."""
    _, inv = index(eri, row_idx_type)
    return inv


def moe_unpermute(permuted, eri, row_idx_type, batch, topk, dtype, probs=None):
    """MoeTokenUnpermute in float64 (TileLang-Ascend operator page, section 4).

    permuted [M, H] (expert outputs in expanded-row order), eri / row_idx_type
    as for moe_dx, probs [batch, topK] or None, all in the storage type
    ``dtype``.  With probs: out[t] = sum_j probs[t, j] * permuted[row(t, j)]
    ([batch, H]), row(t, j) the expanded row of position t*topK + j, summed in
    slot order.  Without: the gather out[p] = permuted[row(p)] ([M, H]).
    """
    M = batch * topk
    inv = _rows_of_positions(eri, row_idx_type)
    rows = decode(np.ascontiguousarray(permuted)[inv], dtype)      # row of each position, [M, H]
    if probs is None:
        return rows
    pr = decode(np.ascontiguousarray(probs), dtype).reshape(batch, topk)
    out = np.zeros((batch, rows.shape[1]), dtype=np.float64)
    for j in range(topk):
        out += pr[:, j:j + 1] * rows[j::topk]
    return out


def moe_unpermute_grad(grad_out, eri, row_idx_type, batch, topk, dtype, permuted=None, probs=None):
    """MoeTokenUnpermuteGrad in float64 (TileLang-Ascend operator page, section 5).

    With probs (and permuted): perm_grad[row(t, j)] = grad_out[t] * probs[t, j]
    ([M, H]) and probs_grad[t, j] = sum_h grad_out[t, h] * permuted[row(t, j), h]
    ([batch, topK]); returns (perm_grad, probs_grad).  Without probs, the
    forward is the gather above and its gradient the scatter
    perm_grad[row(p)] = grad_out[p] (grad_out [M, H]); returns (perm_grad, None).
    """
    M = batch * topk
    inv = _rows_of_positions(eri, row_idx_type)
    g = decode(np.ascontiguousarray(grad_out), dtype)
    perm_grad = np.zeros((M, g.shape[1]), dtype=np.float64)
    if probs is None:
        perm_grad[inv] = g
        return perm_grad, None
    pr = decode(np.ascontiguousarray(probs), dtype).reshape(batch, topk)
    rows = decode(np.ascontiguousarray(permuted)[inv], dtype)
    probs_grad = np.zeros((batch, topk), dtype=np.float64)
    for j in range(topk):
        perm_grad[inv[j::topk]] = g * pr[:, j:j + 1]
        probs_grad[:, j] = np.sum(g * rows[j::topk], axis=1)
    return perm_grad, probs_grad


def case_fwd(case, x, **kw):
    """moe_fwd on a ``synth.Case`` and its forward input x [batch, K]."""
    return moe_fwd(x, case.weight, case.eri, case.group_list, case.batch, case.topk,
                   case.row_idx_type, case.dtype, **kw)


def case_dx_cols(case, cols, **kw):
    return moe_dx_cols(case.grad_y, case.weight, case.eri, case.group_list, case.batch, case.topk,
                       case.row_idx_type, case.dtype, cols, **kw)


def case_colsum(case, cols, **kw):
    return colsum(case.grad_y, case.weight, case.eri, case.group_list, case.batch, case.topk,
                  case.row_idx_type, case.dtype, cols, **kw)


def case_dx(case, mode=SLOT, **kw):
    """moe_dx on a ``synth.Case``."""
    return moe_dx(case.grad_y, case.weight, case.eri, case.group_list, case.batch, case.topk,
                  case.row_idx_type, case.dtype, mode=mode, **kw)


def case_dx_tokens(case, tokens, **kw):
    return moe_dx_tokens(case.grad_y, case.weight, case.eri, case.group_list, case.batch,
                         case.topk, case.row_idx_type, case.dtype, tokens, **kw)
