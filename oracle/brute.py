"""Literal evaluations of the page's formulas in numpy float64 (tiny inputs only).

Test infrastructure; shares nothing with the HIP path.

* ``dx_literal`` is the merged scalar form of the backward of the
  MoeInitRoutingGroupedMatmulGrad design page (§数学定义和公式, the expanded
  scalar formula): for every (b, k), a double sum over all expanded rows i and
  reduction indices n of an indicator [batch(i) == b] times d_y[i,n] times
  W[g(i),k,n].  It walks every (b, i) pair with the indicator instead of
  inverting the routing index, and finds g(i) by scanning the counts.
* ``absdot_literal`` is the same double sum over the magnitudes of the
  terms, |d_y[i,n]| * |W[g(i),k,n]|: the scale of the a-priori error bound
  of an fp32 evaluation of the formula.
* ``forward_literal`` is the forward of the same section:
  expanded_x = Permute(x) and y[i,n] = sum_k expanded_x[i,k] * W[g(i),k,n],
  used for the adjoint identity <d_x, x> = <d_y, y(x)>.
"""
from __future__ import annotations

import numpy as np


def _group_of_rows(group_list: np.ndarray, M: int) -> np.ndarray:
    g_of = np.empty(M, dtype=np.int64)
    start = 0
    for g, c in enumerate(np.asarray(group_list, dtype=np.int64)):
        g_of[start:start + c] = g
        start += c
    if start != M:
        raise ValueError("sum(group_list) != M")
    return g_of


def _original_position(eri: np.ndarray, row_idx_type: int) -> np.ndarray:
    """Original position of every expanded row (type 1 is the scatter form)."""
    eri = np.asarray(eri, dtype=np.int64)
    if row_idx_type == 0:
        return eri.copy()
    pos = np.empty_like(eri)
    for p, i in enumerate(eri):
        pos[i] = p
    return pos


def dx_literal(dy: np.ndarray, W: np.ndarray, eri: np.ndarray, group_list: np.ndarray,
               batch: int, topk: int, row_idx_type: int) -> np.ndarray:
    """d_x[b,k] = sum_i sum_n 1[batch(i)=b] * dy[i,n] * W[g(i),k,n], float64."""
    dy = np.asarray(dy, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    M, N = dy.shape
    G, K, _ = W.shape
    g_of = _group_of_rows(group_list, M)
    pos = _original_position(eri, row_idx_type)
    out = np.zeros((batch, K), dtype=np.float64)
    for b in range(batch):
        for i in range(M):
            indicator = 1.0 if pos[i] // topk == b else 0.0
            if indicator == 0.0:
                continue
            for k in range(K):
                out[b, k] += indicator * float(np.dot(dy[i, :], W[g_of[i], k, :]))
    return out


def absdot_literal(dy: np.ndarray, W: np.ndarray, eri: np.ndarray, group_list: np.ndarray,
                   batch: int, topk: int, row_idx_type: int) -> np.ndarray:
    """sum_i sum_n 1[batch(i)=b] * |dy[i,n]| * |W[g(i),k,n]|, float64, term by term."""
    dy = np.asarray(dy, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    M, N = dy.shape
    G, K, _ = W.shape
    g_of = _group_of_rows(group_list, M)
    pos = _original_position(eri, row_idx_type)
    out = np.zeros((batch, K), dtype=np.float64)
    for b in range(batch):
        for i in range(M):
            if pos[i] // topk != b:
                continue
            for k in range(K):
                for n in range(N):
                    out[b, k] += abs(dy[i, n]) * abs(W[g_of[i], k, n])
    return out


def forward_literal(x: np.ndarray, W: np.ndarray, eri: np.ndarray, group_list: np.ndarray,
                    topk: int, row_idx_type: int) -> np.ndarray:
    """y = GroupedMatmul(Permute(x), W) in float64; x is [batch, K]."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    M = int(np.sum(group_list))
    g_of = _group_of_rows(group_list, M)
    pos = _original_position(eri, row_idx_type)
    expanded_x = x[pos // topk]                     # Permute: row i copies token pos(i)/topK
    y = np.empty((M, W.shape[2]), dtype=np.float64)
    for i in range(M):
        y[i] = expanded_x[i] @ W[g_of[i]]           # sum over k of x[k] * W[g,k,n]
    return y
