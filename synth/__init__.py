"""Seeded synthetic inputs for the fused MoE backward d_x operator.

This module only *constructs inputs*: routing decisions, the expanded-row
order, the routing index in either encoding, per-expert counts and the value
tensors.  It holds none of the operator's arithmetic (no products, no
reductions), so both the HIP path and the CPU oracle can consume its output
without sharing any of the method.

Conventions (MoeInitRoutingGroupedMatmulGrad design page, §数学定义和公式 and
the I/O table of §1.2):

* original position ``p = b * topK + j`` for token ``b`` and routing slot ``j``;
* the forward permute groups expanded rows by expert; inside one expert the
  rows keep ascending ``p`` (a stable sort; the page does not fix this order);
* ``group_list[g]`` is the number of expanded rows of expert ``g`` (counts,
  not a cumulative sum);
* ``row_idx_type == 0``: ``eri[i]`` is the original position of expanded row
  ``i`` (gather, expanded -> original);
  ``row_idx_type == 1``: ``eri[p]`` is the expanded row of original position
  ``p`` (scatter, original -> expanded).

Value tensors are returned in their storage type: ``float32`` and
``float16`` as numpy arrays of that dtype, ``bfloat16`` as ``uint16`` bit
patterns (numpy has no bfloat16).  Rounding from the float32 draw to the
storage type is IEEE round-to-nearest-even.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass
class Case:
    """One synthetic problem instance (host arrays)."""

    batch: int
    topk: int
    G: int
    K: int
    N: int
    dtype: str
    row_idx_type: int
    grad_y: np.ndarray          # [M, N] storage dtype
    weight: np.ndarray          # [G, K, N] storage dtype
    eri: np.ndarray             # int64 [M], encoding given by row_idx_type
    group_list: np.ndarray      # int64 [G] counts
    expert: np.ndarray          # int64 [batch, topK] routing decision (construction record)
    rowpos: np.ndarray          # int64 [batch, topK] expanded row that (b, j) landed in
    name: str = ""
    seed: int = 0

    @property
    def M(self) -> int:
        return self.batch * self.topk


# ----------------------------------------------------------------------------
# rounding to storage types (input construction only)
# ----------------------------------------------------------------------------

_BLOCK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _blocks(n: int):
    return [(s, min(n, s + _BLOCK)) for s in range(0, n, _BLOCK)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return the uint16 bit patterns."""
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def work(se):
        s, e = se
        u = flat[s:e].view(np.uint32)
        r = (u >> 16) & 1          # finite values: u + 0x7FFF + lsb stays below 2^32
        r += 0x7FFF
        r += u
        r >>= 16
        blk = r.astype(np.uint16)
        nan = np.isnan(flat[s:e])
        if nan.any():
            blk[nan] = np.uint16(0x7FC0)
        out[s:e] = blk

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, _blocks(flat.size)))
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        out = np.empty(flat.shape, dtype=np.float16)

        def work(se):
            out[se[0]:se[1]] = flat[se[0]:se[1]].astype(np.float16)

        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, _blocks(flat.size)))
        return out.reshape(np.shape(x))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a storage-typed array to float32 (for test bookkeeping)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    return np.asarray(x).astype(np.float32)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def route_uniform_distinct(rng: np.random.Generator, batch: int, topk: int,
                           experts: Sequence[int]) -> np.ndarray:
    """topK distinct experts per token, uniform over ``experts``; slot order random."""
    experts = np.asarray(experts, dtype=np.int64)
    if topk > len(experts):
        raise ValueError("topK exceeds the number of available experts")
    keys = rng.random((batch, len(experts)))
    pick = np.argsort(keys, axis=1, kind="stable")[:, :topk]
    return experts[pick]


def route_zipf_gumbel(rng: np.random.Generator, batch: int, topk: int, G: int,
                      s: float) -> np.ndarray:
    """topK distinct experts per token by Gumbel-top-k on log p_e, p_e ~ (e+1)^-s.

    Slot order is descending perturbed key."""
    logp = -s * np.log(np.arange(1, G + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(rng.random((batch, G))))
    keys = logp[None, :] + gumbel
    return np.argsort(-keys, axis=1, kind="stable")[:, :topk].astype(np.int64)


def route_heavy(rng: np.random.Generator, batch: int, topk: int, G: int,
                empty: Sequence[int], heavy: int, heavy_rows: int) -> np.ndarray:
    """``heavy_rows`` of the (b, j) pairs, drawn without replacement, go to
    expert ``heavy``; every other pair goes uniformly to the remaining
    non-empty experts.  Duplicate experts inside one token can occur."""
    M = batch * topk
    others = np.array([e for e in range(G) if e not in set(empty) and e != heavy], dtype=np.int64)
    flat = others[rng.integers(0, len(others), size=M)]
    sel = rng.choice(M, size=heavy_rows, replace=False)
    flat[sel] = heavy
    return flat.reshape(batch, topk)


# ----------------------------------------------------------------------------
# assembling a case
# ----------------------------------------------------------------------------

def assemble(expert: np.ndarray, G: int):
    """Expanded-row order of the forward permute (stable by expert).

    Returns (ori, rowpos, group_list): ``ori[i]`` original position of expanded
    row i, ``rowpos[b, j]`` expanded row of (b, j), and per-expert counts."""
    batch, topk = expert.shape
    flat = expert.reshape(-1)
    ori = np.argsort(flat, kind="stable").astype(np.int64)
    rowpos_flat = np.empty_like(ori)
    rowpos_flat[ori] = np.arange(ori.size, dtype=np.int64)
    group_list = np.bincount(flat, minlength=G).astype(np.int64)
    return ori, rowpos_flat.reshape(batch, topk), group_list


def draw_values(seed: int, tensor_id: int, shape, dtype: str, std: float, integer: bool):
    """Values of one tensor, drawn in fixed blocks of 2^22 elements; block t
    uses its own PCG64 stream seeded by (seed, tensor_id, t), so the result
    does not depend on how many threads fill it."""
    n = int(np.prod(shape))
    v = np.empty(n, dtype=np.float32)

    def work(t_se):
        t, (s, e) = t_se
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, t])))
        if integer:
            v[s:e] = rng.integers(-2, 3, size=e - s).astype(np.float32)
        else:
            rng.standard_normal(size=e - s, dtype=np.float32, out=v[s:e])
            if std != 1.0:
                v[s:e] *= np.float32(std)

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, enumerate(_blocks(n))))
    return to_storage(v.reshape(shape), dtype)


def make_case(batch: int, topk: int, G: int, K: int, N: int, dtype: str = "f32", *,
              seed: int = 0, routing: str = "uniform", empty: Sequence[int] = (),
              row_idx_type: int = 0, y_std: float = 1.0, w_std: float = 1.0,
              integer: bool = False, zipf_s: float = 1.1, heavy: Optional[int] = None,
              heavy_rows: int = 0, expert: Optional[np.ndarray] = None,
              name: str = "") -> Case:
    """Build a seeded case.  ``expert`` overrides the routing draw when given."""
    if dtype not in DTYPES:
        raise ValueError(dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    if expert is None:
        avail = [e for e in range(G) if e not in set(empty)]
        if routing == "uniform":
            expert = route_uniform_distinct(rng, batch, topk, avail)
        elif routing == "zipf":
            expert = route_zipf_gumbel(rng, batch, topk, G, zipf_s)
        elif routing == "heavy":
            expert = route_heavy(rng, batch, topk, G, empty, heavy, heavy_rows)
        elif routing == "roundrobin":
            expert = ((np.arange(batch)[:, None] * topk + np.arange(topk)[None, :]) % len(avail))
            expert = np.asarray(avail, dtype=np.int64)[expert]
        else:
            raise ValueError(routing)
    expert = np.asarray(expert, dtype=np.int64)
    ori, rowpos, group_list = assemble(expert, G)
    M = batch * topk
    grad_y = draw_values(seed, 1, (M, N), dtype, y_std, integer)
    weight = draw_values(seed, 2, (G, K, N), dtype, w_std, integer)
    eri = ori.copy() if row_idx_type == 0 else rowpos.reshape(-1).copy()
    return Case(batch=batch, topk=topk, G=G, K=K, N=N, dtype=dtype,
                row_idx_type=row_idx_type, grad_y=grad_y, weight=weight, eri=eri,
                group_list=group_list, expert=expert, rowpos=rowpos, name=name, seed=seed)


# ----------------------------------------------------------------------------
# the five workloads and the white-box matrix
# ----------------------------------------------------------------------------

def forward_input(case: Case, integer: bool = False, std: float = 1.0) -> np.ndarray:
    """The forward's token activations x [batch, K] for a case, in its storage
    type: N(0, std) (or integers in [-2, 2]) from the case's seed, tensor id 3."""
    return draw_values(case.seed, 3, (case.batch, case.K), case.dtype, std, integer)


def _pick_empty(seed: int, G: int, n: int) -> list:
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    return sorted(int(e) for e in rng.choice(G, size=n, replace=False))


CONFIGS = {
    # tiny fp32: batch 64, topK 2, G 4, K 256, N 128; uniform distinct; type 0; N(0,1)
    "tiny_f32": dict(batch=64, topk=2, G=4, K=256, N=128, dtype="f32", seed=1,
                     routing="uniform", row_idx_type=0),
    # decode bf16: batch 16, topK 8, G 16 (4 forced empty), K 7168, N 4096
    "decode_bf16": dict(batch=16, topk=8, G=16, K=7168, N=4096, dtype="bf16", seed=2,
                        routing="uniform", row_idx_type=0, w_std=0.02,
                        empty=_pick_empty(2, 16, 4)),
    # mid bf16: batch 2048, topK 8, G 16, Zipf(1.1) popularity, type 1
    "mid_bf16": dict(batch=2048, topk=8, G=16, K=7168, N=4096, dtype="bf16", seed=3,
                     routing="zipf", row_idx_type=1, w_std=0.02),
    # large fp16: batch 13824, topK 8, G 60, K 7168, N 2048; uniform; type 0
    "large_f16": dict(batch=13824, topk=8, G=60, K=7168, N=2048, dtype="f16", seed=4,
                      routing="uniform", row_idx_type=0, w_std=0.02),
    # large fp32 with 12 empty experts and one expert holding M/4 rows
    "large_f32": dict(batch=13824, topk=8, G=60, K=7168, N=2048, dtype="f32", seed=5,
                      routing="heavy", row_idx_type=0, w_std=0.02),
    # its K/N tail variant
    "large_f32_tail": dict(batch=13824, topk=8, G=60, K=7160, N=2040, dtype="f32", seed=6,
                           routing="heavy", row_idx_type=0, w_std=0.02),
}


def _heavy_setup(cfg: dict) -> dict:
    cfg = dict(cfg)
    if cfg.get("routing") == "heavy":
        G = cfg["G"]
        empty = _pick_empty(cfg["seed"], G, G // 5)
        rest = [e for e in range(G) if e not in empty]
        rng = np.random.Generator(np.random.PCG64(cfg["seed"] + 2000))
        cfg["empty"] = empty
        cfg["heavy"] = int(rest[int(rng.integers(0, len(rest)))])
        cfg["heavy_rows"] = cfg["batch"] * cfg["topk"] // 4
    return cfg


def config_kwargs(name: str, **overrides) -> dict:
    cfg = _heavy_setup(CONFIGS[name])
    cfg.update(overrides)
    return cfg


def make_config(name: str, **overrides) -> Case:
    """One of the named workloads; ``overrides`` can shrink it (e.g. batch=…)."""
    cfg = config_kwargs(name, **overrides)
    return make_case(name=name, **cfg)


# The white-box matrix of the design page (§4.2.1), as (name, kwargs).  The
# page's "ratio" column is read as the fraction of experts that receive tokens.
WHITEBOX = [
    ("one_token_one_expert", dict(batch=1, K=128, N=256, topk=1, G=1)),
    ("one_token_multi_expert", dict(batch=1, K=128, N=256, topk=3, G=3)),
    ("all_tokens_one_expert", dict(batch=128, K=128, N=256, topk=1, G=1)),
    ("general", dict(batch=128, K=128, N=256, topk=3, G=10, empty=(7, 9))),
    ("empty_expert", dict(batch=10, K=128, N=256, topk=2, G=4, empty=(1, 3))),
    ("tails", dict(batch=10, K=128 + 50, N=256 + 30, topk=3, G=4)),
    ("type1", dict(batch=128, K=128, N=256, topk=3, G=10, row_idx_type=1)),
    ("m1", dict(batch=1, topk=1, K=128, N=256, G=1)),
    ("n1", dict(batch=128, K=128, N=1, topk=3, G=4)),
    ("k1", dict(batch=128, K=1, N=256, topk=3, G=4)),
    ("large_tokens", dict(batch=110592, K=128, N=256, topk=2, G=60)),
]
