"""MI355X (gfx950) fused MoE backward producing d_x — Python binding.

A thin ctypes layer over ``libpgg.so`` (built from ``csrc/`` by
``python -m permute_grouped_gemm_amd.build``).  It only marshals arguments:
PyTorch provides device memory and the current stream, and every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing, importing the entry points raises.

    d_x = moe_dx(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type)

computes, for the MoeInitRoutingGroupedMatmulGrad operator (design page,
§数学定义和公式), d_x[b,k] = sum over expanded rows i of token b of
sum_n grad_y[i,n] * weight[g(i),k,n], returned as float32 [batch, K].

    y = moe_fwd(x, weight, expanded_row_idx, group_list, topk, row_idx_type)

is the layer's forward (the same section's forward formulas): Permute then
GroupedMatmul, y[i,n] = sum_k x[p(i) // topK, k] * weight[g(i),k,n], float32
[M, N] in expanded (expert-grouped) row order.

    grad_w = moe_dw(x, grad_y, expanded_row_idx, group_list, topk, row_idx_type)

is the weight gradient (§1.2's separate operator, expanded_x^T · d_y per
expert), float32 [G, K, N], and

    group_list, eri_gather, eri_scatter, expanded_x = moe_routing(expert_ids, G, x)

is MoeInitRouting on the device (§1.1 step 1): the routing tables (and the
permuted x) from the router's choices.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

__all__ = [
    "moe_dx", "moe_dx_noalloc", "workspace_size", "plan", "read_device_error", "debug_tables", "debug_tiles",
    "moe_fwd", "fwd_workspace_size", "fwd_plan", "fwd_kernel_time",
    "moe_dw", "dw_workspace_size", "dw_kernel_time", "moe_routing", "moe_unpermute",
    "moe_unpermute_grad",
    "KernelTimer", "PggError", "lib", "LIB_PATH", "HEADER_PATH",
]

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpgg.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG), "include", "pgg.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP, ERR_MISALIGNED = range(6)
DEV_OK, DEV_GROUP_NEGATIVE, DEV_GROUP_SUM, DEV_INDEX_RANGE, DEV_INDEX_DUP, DEV_EXPERT_RANGE = range(6)
DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class Desc(ctypes.Structure):
    _fields_ = [
        ("grad_y_rows", ctypes.c_int64), ("grad_y_cols", ctypes.c_int64),
        ("weight_groups", ctypes.c_int64), ("weight_rows", ctypes.c_int64),
        ("weight_cols", ctypes.c_int64), ("idx_len", ctypes.c_int64),
        ("group_list_len", ctypes.c_int64), ("batch", ctypes.c_int64), ("topk", ctypes.c_int64),
        ("row_idx_type", ctypes.c_int32), ("grad_y_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class FwdDesc(ctypes.Structure):
    _fields_ = [
        ("x_rows", ctypes.c_int64), ("x_cols", ctypes.c_int64),
        ("weight_groups", ctypes.c_int64), ("weight_rows", ctypes.c_int64),
        ("weight_cols", ctypes.c_int64), ("idx_len", ctypes.c_int64),
        ("group_list_len", ctypes.c_int64), ("batch", ctypes.c_int64), ("topk", ctypes.c_int64),
        ("row_idx_type", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class RoutingDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("topk", ctypes.c_int64), ("experts", ctypes.c_int64),
        ("x_cols", ctypes.c_int64), ("x_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class UnpermuteDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("topk", ctypes.c_int64), ("hidden", ctypes.c_int64),
        ("row_idx_type", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("pad", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("regime", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
        ("tiles_per_chunk", ctypes.c_int32), ("max_tiles", ctypes.c_int32),
        ("max_chunks", ctypes.c_int32), ("ring_rows", ctypes.c_int32),
        ("fused_prep", ctypes.c_int32), ("n_panels", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("panel_cols", ctypes.c_int64),
        ("ring_bytes", ctypes.c_size_t),
        ("table_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved0"}


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


class PggError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        msg = lib().pgg_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded libpgg.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m permute_grouped_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        PD = ctypes.POINTER(Desc)
        L.pgg_moe_dx_workspace_size.argtypes = [PD, ctypes.POINTER(sz)]
        L.pgg_moe_dx.argtypes = [PD, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pgg_moe_dx_read_device_error.argtypes = [vp, vp, ctypes.POINTER(i32), ctypes.POINTER(i64)]
        L.pgg_moe_dx_noalloc.argtypes = [PD, vp, vp, vp, vp, vp, vp, vp]
        L.pgg_moe_dx_debug_tables.argtypes = [PD, vp, vp, vp, vp]
        L.pgg_moe_dx_debug_tiles.argtypes = [PD, vp, vp, vp, i32, ctypes.POINTER(i32)]
        L.pgg_moe_dx_plan.argtypes = [PD, ctypes.POINTER(Plan)]
        L.pgg_moe_dx_kernel_time.argtypes = [PD, vp, vp, vp, vp, vp, vp, sz, vp, i32, i32,
                                              ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
        PF = ctypes.POINTER(FwdDesc)
        L.pgg_moe_fwd_workspace_size.argtypes = [PF, ctypes.POINTER(sz)]
        L.pgg_moe_fwd.argtypes = [PF, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pgg_moe_fwd_plan.argtypes = [PF, ctypes.POINTER(Plan)]
        L.pgg_moe_fwd_kernel_time.argtypes = [PF, vp, vp, vp, vp, vp, vp, sz, vp, i32,
                                               ctypes.POINTER(ctypes.c_double)]
        L.pgg_moe_dw_workspace_size.argtypes = [PF, ctypes.POINTER(sz)]
        L.pgg_moe_dw.argtypes = [PF, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pgg_moe_dw_kernel_time.argtypes = [PF, vp, vp, vp, vp, vp, vp, sz, vp, i32,
                                              ctypes.POINTER(ctypes.c_double)]
        PR = ctypes.POINTER(RoutingDesc)
        L.pgg_moe_routing_workspace_size.argtypes = [PR, ctypes.POINTER(sz)]
        L.pgg_moe_routing.argtypes = [PR, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        PU = ctypes.POINTER(UnpermuteDesc)
        L.pgg_moe_unpermute_workspace_size.argtypes = [PU, ctypes.POINTER(sz)]
        L.pgg_moe_unpermute.argtypes = [PU, vp, vp, vp, vp, vp, sz, vp]
        L.pgg_moe_unpermute_grad.argtypes = [PU, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pgg_timing_begin.argtypes = [i32]
        L.pgg_timing_end.argtypes = [ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)]
        L.pgg_status_string.argtypes = [ctypes.c_int]
        L.pgg_status_string.restype = ctypes.c_char_p
        L.pgg_device_error_string.argtypes = [i32]
        L.pgg_device_error_string.restype = ctypes.c_char_p
        for f in ("pgg_moe_dx_workspace_size", "pgg_moe_dx", "pgg_moe_dx_noalloc",
                  "pgg_moe_dx_read_device_error",
                  "pgg_moe_dx_debug_tables", "pgg_moe_dx_debug_tiles", "pgg_moe_dx_plan",
                  "pgg_moe_dx_kernel_time", "pgg_moe_fwd_workspace_size", "pgg_moe_fwd",
                  "pgg_moe_fwd_plan", "pgg_moe_fwd_kernel_time", "pgg_moe_dw_workspace_size",
                  "pgg_moe_dw", "pgg_moe_dw_kernel_time", "pgg_moe_routing_workspace_size",
                  "pgg_moe_routing", "pgg_moe_unpermute_workspace_size", "pgg_moe_unpermute",
                  "pgg_moe_unpermute_grad",
                  "pgg_timing_begin", "pgg_timing_end"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/pgg.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pgg_\w+)\s*\(", text, re.M)))


def _check(status: int, where: str):
    if status != OK:
        raise PggError(status, where)


def make_desc(grad_y_shape, weight_shape, idx_len, group_list_len, batch, topk, row_idx_type,
              grad_y_dtype, weight_dtype) -> Desc:
    if len(grad_y_shape) != 2 or len(weight_shape) != 3:
        raise PggError(ERR_INVALID_ARG, "rank")
    d = Desc()
    d.grad_y_rows, d.grad_y_cols = (int(v) for v in grad_y_shape)
    d.weight_groups, d.weight_rows, d.weight_cols = (int(v) for v in weight_shape)
    d.idx_len = int(idx_len)
    d.group_list_len = int(group_list_len)
    d.batch = int(batch)
    d.topk = int(topk)
    d.row_idx_type = int(row_idx_type)
    d.grad_y_dtype = grad_y_dtype
    d.weight_dtype = weight_dtype
    d.reserved = 0
    return d


def _desc_from_tensors(grad_y, weight, eri, group_list, batch, topk, row_idx_type) -> Desc:
    if eri.dim() != 1 or group_list.dim() != 1:
        raise PggError(ERR_INVALID_ARG, "rank")
    if eri.dtype != torch.int64 or group_list.dtype != torch.int64:
        raise PggError(ERR_INVALID_ARG, "index dtype")
    gy = DTYPE_CODE.get(grad_y.dtype, -1)
    wt = DTYPE_CODE.get(weight.dtype, -1)
    return make_desc(grad_y.shape, weight.shape, eri.shape[0], group_list.shape[0], batch, topk,
                     row_idx_type, gy, wt)


def workspace_size_desc(d: Desc) -> int:
    n = ctypes.c_size_t()
    _check(lib().pgg_moe_dx_workspace_size(ctypes.byref(d), ctypes.byref(n)), "workspace_size")
    return n.value


def plan_desc(d: Desc) -> dict:
    p = Plan()
    _check(lib().pgg_moe_dx_plan(ctypes.byref(d), ctypes.byref(p)), "plan")
    return p.as_dict()


def workspace_size(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type=0) -> int:
    return workspace_size_desc(_desc_from_tensors(grad_y, weight, expanded_row_idx, group_list,
                                                  batch, topk, row_idx_type))


def plan(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type=0) -> dict:
    return plan_desc(_desc_from_tensors(grad_y, weight, expanded_row_idx, group_list, batch, topk,
                                        row_idx_type))


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_inputs(*tensors):
    dev = tensors[0].device
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous() or t.device != dev:
            raise PggError(ERR_INVALID_ARG, "inputs must be contiguous tensors on one GPU")


def _check_workspace(workspace, dev):
    if workspace.device != dev or not workspace.is_contiguous():
        raise PggError(ERR_INVALID_ARG, "workspace must be a contiguous tensor on the inputs' GPU")


def _check_out(out, batch, weight, dev):
    if (out.dtype != torch.float32 or not out.is_contiguous() or out.device != dev
            or tuple(out.shape) != (int(batch), int(weight.shape[1]))):
        raise PggError(ERR_INVALID_ARG, "out must be a contiguous float32 [batch, K] tensor on the inputs' GPU")


def moe_dx(grad_y: torch.Tensor, weight: torch.Tensor, expanded_row_idx: torch.Tensor,
           group_list: torch.Tensor, batch: int, topk: int, row_idx_type: int = 0, *,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Fused backward: float32 d_x [batch, K] (asynchronous on the current stream).

    grad_y [M, N] and weight [G, K, N] share one of float32 / float16 /
    bfloat16; expanded_row_idx [M] and group_list [G] are int64; all on one
    GPU.  ``workspace`` (uint8, at least ``workspace_size(...)`` bytes,
    256-byte aligned) and ``out`` may be passed to avoid allocations."""
    d = _desc_from_tensors(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type)
    _check_inputs(grad_y, weight, expanded_row_idx, group_list)
    need = workspace_size_desc(d)
    dev = grad_y.device
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((int(batch), int(weight.shape[1])), dtype=torch.float32, device=dev)
    _check_out(out, batch, weight, dev)
    _check_workspace(workspace, dev)
    st = lib().pgg_moe_dx(ctypes.byref(d), grad_y.data_ptr(), weight.data_ptr(),
                          expanded_row_idx.data_ptr(), group_list.data_ptr(), out.data_ptr(),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream_handle(stream))
    _check(st, "pgg_moe_dx")
    return out


def moe_dx_noalloc(grad_y: torch.Tensor, weight: torch.Tensor, expanded_row_idx: torch.Tensor,
                   group_list: torch.Tensor, batch: int, topk: int, row_idx_type: int = 0, *,
                   out: torch.Tensor, device_error: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """pgg_moe_dx_noalloc: the fused backward into ``out`` (float32 [batch, K])
    with the library's fixed device scratch as workspace; ``device_error``
    (optional int64 [2] on the GPU) receives [code, detail] of this call."""
    d = _desc_from_tensors(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type)
    _check_inputs(grad_y, weight, expanded_row_idx, group_list)
    _check_out(out, batch, weight, grad_y.device)
    if device_error is not None and (device_error.dtype != torch.int64 or device_error.numel() < 2
                                     or device_error.device != grad_y.device):
        raise PggError(ERR_INVALID_ARG, "device_error must be an int64 tensor of 2 elements on the inputs' GPU")
    st = lib().pgg_moe_dx_noalloc(ctypes.byref(d), grad_y.data_ptr(), weight.data_ptr(),
                                  expanded_row_idx.data_ptr(), group_list.data_ptr(), out.data_ptr(),
                                  None if device_error is None else device_error.data_ptr(),
                                  _stream_handle(stream))
    _check(st, "pgg_moe_dx_noalloc")
    return out


def _ws_bytes(workspace):
    return workspace.numel() * workspace.element_size()


def _check_tables_workspace(workspace, d, dev):
    """The debug readers copy index tables out of ``workspace``: it must be the
    inputs' GPU's workspace of a call with this descriptor (all its tables)."""
    if not workspace.is_cuda:
        raise PggError(ERR_INVALID_ARG, "workspace must be a GPU tensor")
    _check_workspace(workspace, dev)
    if _ws_bytes(workspace) < plan_desc(d)["table_bytes"]:
        raise PggError(ERR_WORKSPACE_TOO_SMALL, "workspace smaller than this call's index tables")


# the device error word sits in the workspace's first 64 bytes
_WS_HEADER_BYTES = 64


def read_device_error(workspace: torch.Tensor, stream=None) -> Tuple[int, int]:
    if not workspace.is_cuda or not workspace.is_contiguous() or _ws_bytes(workspace) < _WS_HEADER_BYTES:
        raise PggError(ERR_INVALID_ARG, "workspace must be a contiguous GPU tensor of a call's workspace")
    code = ctypes.c_int32()
    detail = ctypes.c_int64()
    _check(lib().pgg_moe_dx_read_device_error(workspace.data_ptr(), _stream_handle(stream),
                                              ctypes.byref(code), ctypes.byref(detail)),
           "read_device_error")
    return code.value, detail.value


def debug_tables(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type,
                 workspace, stream=None):
    """(inv, ori) int32 host tensors built by the last call on ``workspace``."""
    d = _desc_from_tensors(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type)
    _check_tables_workspace(workspace, d, grad_y.device)
    M = d.grad_y_rows
    inv = torch.empty(M, dtype=torch.int32)
    ori = torch.empty(M, dtype=torch.int32)
    _check(lib().pgg_moe_dx_debug_tables(ctypes.byref(d), workspace.data_ptr(),
                                         _stream_handle(stream), inv.data_ptr(), ori.data_ptr()),
           "debug_tables")
    return inv, ori


def debug_tiles(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type,
                workspace, stream=None):
    """m-tile table [(expert, first row, rows)] built by the last call on ``workspace``."""
    d = _desc_from_tensors(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type)
    _check_tables_workspace(workspace, d, grad_y.device)
    cap = plan_desc(d)["max_tiles"]
    buf = torch.empty(3 * cap, dtype=torch.int32)
    n = ctypes.c_int32()
    _check(lib().pgg_moe_dx_debug_tiles(ctypes.byref(d), workspace.data_ptr(), _stream_handle(stream),
                                        buf.data_ptr(), cap, ctypes.byref(n)), "debug_tiles")
    return buf[: 3 * n.value].reshape(-1, 3)


def kernel_time(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type=0, *,
                which: str = "produce", repeats: int = 10, out=None, workspace=None,
                stream=None) -> Tuple[float, int]:
    """(average ms of one launch, launches per call) of the producer
    (``which="produce"``) or the consumer (``"consume"``), launched back to
    back between two HIP events after one full call (pgg_moe_dx_kernel_time)."""
    d = _desc_from_tensors(grad_y, weight, expanded_row_idx, group_list, batch, topk, row_idx_type)
    _check_inputs(grad_y, weight, expanded_row_idx, group_list)
    dev = grad_y.device
    if workspace is None:
        workspace = torch.empty(workspace_size_desc(d), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    if out is None:
        out = torch.empty((int(batch), int(weight.shape[1])), dtype=torch.float32, device=dev)
    _check_out(out, batch, weight, dev)
    avg = ctypes.c_double()
    n = ctypes.c_int32()
    w = {"produce": 0, "consume": 1}[which]
    _check(lib().pgg_moe_dx_kernel_time(ctypes.byref(d), grad_y.data_ptr(), weight.data_ptr(),
                                        expanded_row_idx.data_ptr(), group_list.data_ptr(),
                                        out.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream_handle(stream), w, int(repeats), ctypes.byref(avg),
                                        ctypes.byref(n)), "kernel_time")
    return avg.value, n.value


# ---------------------------------------------------------------- forward

def make_fwd_desc(x_shape, weight_shape, idx_len, group_list_len, batch, topk, row_idx_type,
                  x_dtype, weight_dtype) -> FwdDesc:
    if len(x_shape) != 2 or len(weight_shape) != 3:
        raise PggError(ERR_INVALID_ARG, "rank")
    d = FwdDesc()
    d.x_rows, d.x_cols = (int(v) for v in x_shape)
    d.weight_groups, d.weight_rows, d.weight_cols = (int(v) for v in weight_shape)
    d.idx_len = int(idx_len)
    d.group_list_len = int(group_list_len)
    d.batch = int(batch)
    d.topk = int(topk)
    d.row_idx_type = int(row_idx_type)
    d.x_dtype = x_dtype
    d.weight_dtype = weight_dtype
    d.reserved = 0
    return d


def _fwd_desc_from_tensors(x, weight, eri, group_list, topk, row_idx_type) -> FwdDesc:
    if eri.dim() != 1 or group_list.dim() != 1 or x.dim() != 2:
        raise PggError(ERR_INVALID_ARG, "rank")
    if eri.dtype != torch.int64 or group_list.dtype != torch.int64:
        raise PggError(ERR_INVALID_ARG, "index dtype")
    return make_fwd_desc(x.shape, weight.shape, eri.shape[0], group_list.shape[0], x.shape[0], topk,
                         row_idx_type, DTYPE_CODE.get(x.dtype, -1), DTYPE_CODE.get(weight.dtype, -1))


def fwd_workspace_size_desc(d: FwdDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().pgg_moe_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n)), "fwd_workspace_size")
    return n.value


def fwd_workspace_size(x, weight, expanded_row_idx, group_list, topk, row_idx_type=0) -> int:
    return fwd_workspace_size_desc(_fwd_desc_from_tensors(x, weight, expanded_row_idx, group_list,
                                                          topk, row_idx_type))


def fwd_plan(x, weight, expanded_row_idx, group_list, topk, row_idx_type=0) -> dict:
    d = _fwd_desc_from_tensors(x, weight, expanded_row_idx, group_list, topk, row_idx_type)
    p = Plan()
    _check(lib().pgg_moe_fwd_plan(ctypes.byref(d), ctypes.byref(p)), "fwd_plan")
    return p.as_dict()


def _fwd_buffers(d, x, weight, out, workspace):
    dev = x.device
    if workspace is None:
        workspace = torch.empty(fwd_workspace_size_desc(d), dtype=torch.uint8, device=dev)
    shape = (int(d.batch * d.topk), int(weight.shape[2]))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    if (out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape
            or out.device != dev):
        raise PggError(ERR_INVALID_ARG, "out must be a contiguous float32 [M, N] tensor on the inputs' GPU")
    _check_workspace(workspace, dev)
    return out, workspace


def moe_fwd(x: torch.Tensor, weight: torch.Tensor, expanded_row_idx: torch.Tensor,
            group_list: torch.Tensor, topk: int, row_idx_type: int = 0, *,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """Forward Permute + GroupedMatmul: float32 y [batch*topk, N] (asynchronous).

    x [batch, K] and weight [G, K, N] share one of float32 / float16 /
    bfloat16; expanded_row_idx [batch*topk] and group_list [G] are int64."""
    d = _fwd_desc_from_tensors(x, weight, expanded_row_idx, group_list, topk, row_idx_type)
    _check_inputs(x, weight, expanded_row_idx, group_list)
    out, workspace = _fwd_buffers(d, x, weight, out, workspace)
    st = lib().pgg_moe_fwd(ctypes.byref(d), x.data_ptr(), weight.data_ptr(),
                           expanded_row_idx.data_ptr(), group_list.data_ptr(), out.data_ptr(),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream_handle(stream))
    _check(st, "pgg_moe_fwd")
    return out


def fwd_kernel_time(x, weight, expanded_row_idx, group_list, topk, row_idx_type=0, *,
                    repeats: int = 10, out=None, workspace=None, stream=None) -> float:
    """Average ms of one launch of the forward's grouped-matmul kernel, launched
    back to back after one full call (pgg_moe_fwd_kernel_time)."""
    d = _fwd_desc_from_tensors(x, weight, expanded_row_idx, group_list, topk, row_idx_type)
    _check_inputs(x, weight, expanded_row_idx, group_list)
    out, workspace = _fwd_buffers(d, x, weight, out, workspace)
    avg = ctypes.c_double()
    _check(lib().pgg_moe_fwd_kernel_time(ctypes.byref(d), x.data_ptr(), weight.data_ptr(),
                                         expanded_row_idx.data_ptr(), group_list.data_ptr(),
                                         out.data_ptr(), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(),
                                         _stream_handle(stream), int(repeats), ctypes.byref(avg)),
           "fwd_kernel_time")
    return avg.value


# ---------------------------------------------------------------- weight gradient

def _dw_desc_from_tensors(x, grad_y, eri, group_list, topk, row_idx_type) -> FwdDesc:
    if x.dim() != 2 or grad_y.dim() != 2 or eri.dim() != 1 or group_list.dim() != 1:
        raise PggError(ERR_INVALID_ARG, "rank")
    if eri.dtype != torch.int64 or group_list.dtype != torch.int64:
        raise PggError(ERR_INVALID_ARG, "index dtype")
    if grad_y.shape[0] != x.shape[0] * int(topk):
        raise PggError(ERR_INVALID_ARG, "grad_y must be [batch*topk, N]")
    G = group_list.shape[0]
    return make_fwd_desc(x.shape, (G, x.shape[1], grad_y.shape[1]), eri.shape[0], G, x.shape[0], topk,
                         row_idx_type, DTYPE_CODE.get(x.dtype, -1), DTYPE_CODE.get(grad_y.dtype, -1))


def dw_workspace_size(x, grad_y, expanded_row_idx, group_list, topk, row_idx_type=0) -> int:
    d = _dw_desc_from_tensors(x, grad_y, expanded_row_idx, group_list, topk, row_idx_type)
    n = ctypes.c_size_t()
    _check(lib().pgg_moe_dw_workspace_size(ctypes.byref(d), ctypes.byref(n)), "dw_workspace_size")
    return n.value


def _dw_buffers(d, x, out, workspace):
    dev = x.device
    if workspace is None:
        n = ctypes.c_size_t()
        _check(lib().pgg_moe_dw_workspace_size(ctypes.byref(d), ctypes.byref(n)), "dw_workspace_size")
        workspace = torch.empty(n.value, dtype=torch.uint8, device=dev)
    shape = (int(d.weight_groups), int(d.weight_rows), int(d.weight_cols))
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    if (out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape
            or out.device != dev):
        raise PggError(ERR_INVALID_ARG, "out must be a contiguous float32 [G, K, N] tensor on the inputs' GPU")
    _check_workspace(workspace, dev)
    return out, workspace


def moe_dw(x: torch.Tensor, grad_y: torch.Tensor, expanded_row_idx: torch.Tensor,
           group_list: torch.Tensor, topk: int, row_idx_type: int = 0, *,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Weight gradient: float32 grad_w [G, K, N], grad_w[g] = (x rows of expert
    g's expanded rows)^T · grad_y[those rows] (asynchronous).  x [batch, K] and
    grad_y [batch*topk, N] share one of float32 / float16 / bfloat16."""
    d = _dw_desc_from_tensors(x, grad_y, expanded_row_idx, group_list, topk, row_idx_type)
    _check_inputs(x, grad_y, expanded_row_idx, group_list)
    out, workspace = _dw_buffers(d, x, out, workspace)
    st = lib().pgg_moe_dw(ctypes.byref(d), x.data_ptr(), grad_y.data_ptr(),
                          expanded_row_idx.data_ptr(), group_list.data_ptr(), out.data_ptr(),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream_handle(stream))
    _check(st, "pgg_moe_dw")
    return out


def dw_kernel_time(x, grad_y, expanded_row_idx, group_list, topk, row_idx_type=0, *,
                   repeats: int = 10, out=None, workspace=None, stream=None) -> float:
    """Average ms of one launch of the weight-gradient kernel, back to back
    after one full call (pgg_moe_dw_kernel_time)."""
    d = _dw_desc_from_tensors(x, grad_y, expanded_row_idx, group_list, topk, row_idx_type)
    _check_inputs(x, grad_y, expanded_row_idx, group_list)
    out, workspace = _dw_buffers(d, x, out, workspace)
    avg = ctypes.c_double()
    _check(lib().pgg_moe_dw_kernel_time(ctypes.byref(d), x.data_ptr(), grad_y.data_ptr(),
                                        expanded_row_idx.data_ptr(), group_list.data_ptr(),
                                        out.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream_handle(stream), int(repeats), ctypes.byref(avg)),
           "dw_kernel_time")
    return avg.value


# ---------------------------------------------------------------- routing

def make_routing_desc(batch, topk, experts, x_cols=0, x_dtype=0) -> RoutingDesc:
    d = RoutingDesc()
    d.batch, d.topk, d.experts, d.x_cols = int(batch), int(topk), int(experts), int(x_cols)
    d.x_dtype = int(x_dtype)
    d.reserved = 0
    return d


def routing_workspace_size_desc(d: RoutingDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().pgg_moe_routing_workspace_size(ctypes.byref(d), ctypes.byref(n)),
           "routing_workspace_size")
    return n.value


def moe_routing(expert_ids: torch.Tensor, experts: int, x: Optional[torch.Tensor] = None, *,
                gather: bool = True, scatter: bool = True, workspace=None, stream=None):
    """MoeInitRouting on the device: (group_list [G], eri_gather [M] or None,
    eri_scatter [M] or None, expanded_x [M, K] or None) from expert_ids
    [batch, topk] int64 (asynchronous).  With x [batch, K], expanded_x is the
    permuted copy of x in expanded-row order."""
    if expert_ids.dim() != 2 or expert_ids.dtype != torch.int64:
        raise PggError(ERR_INVALID_ARG, "expert_ids must be an int64 [batch, topk] tensor")
    if not expert_ids.is_cuda or not expert_ids.is_contiguous():
        raise PggError(ERR_INVALID_ARG, "expert_ids must be a contiguous GPU tensor")
    batch, topk = expert_ids.shape
    K, xd = 0, 0
    if x is not None:
        if x.dim() != 2 or x.shape[0] != batch or x.device != expert_ids.device or not x.is_contiguous():
            raise PggError(ERR_INVALID_ARG, "x must be a contiguous [batch, K] tensor on expert_ids' GPU")
        K, xd = x.shape[1], DTYPE_CODE.get(x.dtype, -1)
    d = make_routing_desc(batch, topk, experts, K, xd)
    dev = expert_ids.device
    if workspace is None:
        workspace = torch.empty(routing_workspace_size_desc(d), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    M = batch * topk
    gl = torch.empty(int(experts), dtype=torch.int64, device=dev)
    eg = torch.empty(M, dtype=torch.int64, device=dev) if gather else None
    es = torch.empty(M, dtype=torch.int64, device=dev) if scatter else None
    ex = torch.empty((M, K), dtype=x.dtype, device=dev) if x is not None else None
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib().pgg_moe_routing(ctypes.byref(d), expert_ids.data_ptr(), ptr(x), gl.data_ptr(), ptr(eg),
                               ptr(es), ptr(ex), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(st, "pgg_moe_routing")
    return gl, eg, es, ex


# ---------------------------------------------------------------- unpermute

def make_unpermute_desc(batch, topk, hidden, row_idx_type, dtype) -> UnpermuteDesc:
    d = UnpermuteDesc()
    d.batch, d.topk, d.hidden = int(batch), int(topk), int(hidden)
    d.row_idx_type, d.dtype, d.reserved, d.pad = int(row_idx_type), int(dtype), 0, 0
    return d


def _check_value(t, shape, like, name):
    """t: a contiguous 2-D tensor of like's dtype on like's GPU (of `shape` when given)."""
    if (t.dim() != 2 or not t.is_contiguous() or t.device != like.device or not t.is_cuda
            or t.dtype != like.dtype or (shape is not None and tuple(t.shape) != shape)):
        want = "" if shape is None else f" {list(shape)}"
        raise PggError(ERR_INVALID_ARG, f"{name} must be a contiguous{want} {like.dtype} GPU tensor "
                                        f"on {like.device}")


def _check_index(t, n, like):
    if t.dtype != torch.int64 or t.dim() != 1 or t.numel() != n or not t.is_contiguous() \
            or t.device != like.device:
        raise PggError(ERR_INVALID_ARG, f"expanded_row_idx must be a contiguous int64 [{n}] tensor "
                                        f"on {like.device}")


def _unpermute_ws(d, dev, workspace):
    if workspace is not None:
        _check_workspace(workspace, dev)
        return workspace
    n = ctypes.c_size_t()
    _check(lib().pgg_moe_unpermute_workspace_size(ctypes.byref(d), ctypes.byref(n)),
           "unpermute_workspace_size")
    return torch.empty(n.value, dtype=torch.uint8, device=dev)


def moe_unpermute(permuted: torch.Tensor, expanded_row_idx: torch.Tensor, batch: int, topk: int,
                  row_idx_type: int = 0, probs: Optional[torch.Tensor] = None, *, workspace=None,
                  stream=None) -> torch.Tensor:
    """MoeTokenUnpermute: with probs [batch, topk], out [batch, H] = sum over
    slots of probs * the token's expert rows; without, the gather [M, H].
    permuted [batch*topk, H]; results in permuted's dtype (fp32 arithmetic)."""
    M = int(batch) * int(topk)
    _check_value(permuted, None, permuted, "permuted")
    H = permuted.shape[1]
    _check_value(permuted, (M, H), permuted, "permuted")
    _check_index(expanded_row_idx, M, permuted)
    if probs is not None:
        _check_value(probs, (int(batch), int(topk)), permuted, "probs")
    d = make_unpermute_desc(batch, topk, H, row_idx_type, DTYPE_CODE.get(permuted.dtype, -1))
    shape = (int(batch), H) if probs is not None else (int(batch) * int(topk), H)
    out = torch.empty(shape, dtype=permuted.dtype, device=permuted.device)
    ws = _unpermute_ws(d, permuted.device, workspace)
    st = lib().pgg_moe_unpermute(ctypes.byref(d), permuted.data_ptr(), expanded_row_idx.data_ptr(),
                                 None if probs is None else probs.data_ptr(), out.data_ptr(),
                                 ws.data_ptr(), _ws_bytes(ws), _stream_handle(stream))
    _check(st, "pgg_moe_unpermute")
    return out


def moe_unpermute_grad(grad: torch.Tensor, expanded_row_idx: torch.Tensor, batch: int, topk: int,
                       row_idx_type: int = 0, permuted: Optional[torch.Tensor] = None,
                       probs: Optional[torch.Tensor] = None, *, workspace=None, stream=None):
    """MoeTokenUnpermuteGrad: (perm_grad [M, H], probs_grad [batch, topk] or
    None).  With probs, grad is [batch, H] and permuted is needed; without,
    grad is [M, H] and perm_grad its scatter back to expanded rows."""
    M = int(batch) * int(topk)
    _check_value(grad, None, grad, "grad")
    H = grad.shape[1]
    _check_value(grad, (int(batch) if probs is not None else M, H), grad, "grad")
    _check_index(expanded_row_idx, M, grad)
    if probs is not None:
        _check_value(probs, (int(batch), int(topk)), grad, "probs")
        if permuted is None:
            raise PggError(ERR_INVALID_ARG, "permuted is needed with probs")
        _check_value(permuted, (M, H), grad, "permuted")
    d = make_unpermute_desc(batch, topk, H, row_idx_type, DTYPE_CODE.get(grad.dtype, -1))
    perm_grad = torch.empty((M, H), dtype=grad.dtype, device=grad.device)
    probs_grad = (torch.empty((int(batch), int(topk)), dtype=grad.dtype, device=grad.device)
                  if probs is not None else None)
    ws = _unpermute_ws(d, grad.device, workspace)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib().pgg_moe_unpermute_grad(ctypes.byref(d), ptr(permuted), grad.data_ptr(),
                                      expanded_row_idx.data_ptr(), ptr(probs), perm_grad.data_ptr(),
                                      ptr(probs_grad), ws.data_ptr(), _ws_bytes(ws), _stream_handle(stream))
    _check(st, "pgg_moe_unpermute_grad")
    return perm_grad, probs_grad


class KernelTimer:
    """Per-kernel HIP-event timing of pgg_moe_dx / pgg_moe_fwd calls made inside the block."""

    def __init__(self, capacity: int = 4096):
        self.capacity = capacity
        self.result = {}

    def __enter__(self):
        _check(lib().pgg_timing_begin(self.capacity), "timing_begin")
        return self

    def __exit__(self, *exc):
        out = (KernelTime * 64)()
        n = ctypes.c_int32()
        st = lib().pgg_timing_end(out, 64, ctypes.byref(n))
        self.result = {out[i].name.decode(): (out[i].launches, out[i].total_ms)
                       for i in range(min(n.value, 64))}
        if exc[0] is None:
            _check(st, "timing_end")
        return False
