"""Helpers for the GPU tests: move a synth.Case to the device and run the
library on it (through the C-ABI binding)."""
import numpy as np
import torch

import permute_grouped_gemm_amd as pgg


def to_torch(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr))


def upload(case, device="cuda"):
    gy = to_torch(case.grad_y, case.dtype).to(device)
    w = to_torch(case.weight, case.dtype).to(device)
    eri = torch.from_numpy(np.ascontiguousarray(case.eri, dtype=np.int64)).to(device)
    gl = torch.from_numpy(np.ascontiguousarray(case.group_list, dtype=np.int64)).to(device)
    return gy, w, eri, gl


def run(case, tensors=None, workspace=None, out=None, check_error=True):
    """d_x from the HIP path as a float32 numpy array (synchronises)."""
    gy, w, eri, gl = tensors if tensors is not None else upload(case)
    if workspace is None:
        workspace = torch.empty(pgg.workspace_size(gy, w, eri, gl, case.batch, case.topk,
                                                   case.row_idx_type),
                                dtype=torch.uint8, device=gy.device)
    dx = pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type,
                    workspace=workspace, out=out)
    torch.cuda.synchronize()
    if check_error:
        code, detail = pgg.read_device_error(workspace)
        assert code == pgg.DEV_OK, (code, detail)
    return dx.cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
