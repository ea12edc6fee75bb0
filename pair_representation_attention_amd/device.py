"""Device-memory helpers around the ctypes binding (argument marshalling only).

Uploads host arrays as torch device tensors of the library's element type,
allocates outputs and the caller-owned workspace, and calls the C entry
points.  All arithmetic happens in the HIP library.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import lib

BF16 = "bf16"
F32 = "f32"


def _torch():
    import torch
    return torch


def dtype_code(dtype: str) -> int:
    return lib.PAIRATTN_BF16 if dtype == BF16 else lib.PAIRATTN_F32


def torch_dtype(dtype: str):
    torch = _torch()
    return torch.bfloat16 if dtype == BF16 else torch.float32


def to_device(a: Optional[np.ndarray], dtype: str, device="cuda"):
    """float32 host values (bf16-exact for the bf16 path) -> device tensor."""
    if a is None:
        return None
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch_dtype(dtype)).contiguous()


def mask_to_device(m: Optional[np.ndarray], device="cuda"):
    if m is None:
        return None
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(m, dtype=np.uint8)).to(device)


def alloc_workspace(nbytes: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def make_params(p, dtype: str, workspace_bytes: int = 0, device="cuda") -> lib.Params:
    """Upload an ``inputs.Params`` weight set; attach a workspace of the given size."""
    tens = {}
    for name in lib.Params.NAMES:
        v = getattr(p, name, None)
        tens[name] = to_device(v, dtype, device) if v is not None else None
    ws = alloc_workspace(workspace_bytes, device) if workspace_bytes else None
    return lib.Params(dtype_code(dtype), eps=p.eps, workspace=ws, **tens)


# ----------------------------------------------------------------------------
# one-call wrappers used by tests, the smoke check and the benchmark
# ----------------------------------------------------------------------------
class TriRunner:
    """Device-resident triangle-attention problem (inputs uploaded once)."""

    def __init__(self, z: np.ndarray, mask: Optional[np.ndarray], params, H: int, dtype: str, d: int = 32,
                 device="cuda"):
        torch = _torch()
        self.I, _, self.c = z.shape
        self.H, self.d, self.dtype = H, d, dtype
        self.z = to_device(z, dtype, device)
        self.mask = mask_to_device(mask, device)
        nbytes = lib.pairattn_tri_workspace_bytes(self.I, self.c, H, d, dtype_code(dtype))
        self.params = make_params(params, dtype, nbytes, device)
        self.out = torch.empty_like(self.z)

    def __call__(self, orientation: int, stream=None):
        lib.pairattn_tri_fwd(self.z, self.mask, self.params, self.out, self.I, self.c, self.H, self.d,
                             orientation, stream)
        return self.out


class TriChunkedRunner:
    """Triangle attention of a device-resident Z in blocks of rows (START)
    or columns (END): pairattn_tri_chunked_fwd."""

    def __init__(self, z_dev, mask_dev, params, H: int, dtype: str, block: int, d: int = 32, device="cuda"):
        torch = _torch()
        self.I, _, self.c = z_dev.shape
        self.H, self.d, self.dtype, self.block = H, d, dtype, block
        self.z = z_dev
        self.mask = mask_dev
        self.workspace_bytes = lib.pairattn_tri_chunked_workspace_bytes(self.I, self.c, H, d, dtype_code(dtype), block)
        self.params = make_params(params, dtype, self.workspace_bytes, device)
        self.out = torch.empty_like(self.z)

    def __call__(self, orientation: int, stream=None):
        lib.pairattn_tri_chunked_fwd(self.z, self.mask, self.params, self.out, self.I, self.c, self.H, self.d,
                                     orientation, self.block, stream)
        return self.out


class MsaRunner:
    def __init__(self, m: np.ndarray, z: np.ndarray, mask: Optional[np.ndarray], params, H: int, dtype: str,
                 d: int = 32, device="cuda"):
        torch = _torch()
        self.S, self.I, self.c_m = m.shape
        self.c_z = z.shape[-1]
        self.H, self.d, self.dtype = H, d, dtype
        self.m = to_device(m, dtype, device)
        self.z = to_device(z, dtype, device)
        self.mask = mask_to_device(mask, device)
        nbytes = lib.pairattn_msa_workspace_bytes(self.S, self.I, self.c_m, self.c_z, H, d, dtype_code(dtype))
        self.params = make_params(params, dtype, nbytes, device)
        self.out = torch.empty_like(self.m)

    def __call__(self, stream=None):
        lib.pairattn_msa_row_fwd(self.m, self.z, self.mask, self.params, self.out, self.S, self.I, self.c_m,
                                 self.c_z, self.H, self.d, stream)
        return self.out


class RowsRunner:
    """Starting-node attention for R query rows of a larger Z with the bias
    of the whole Z (computed by pairattn_tri_bias)."""

    def __init__(self, z_full_dev, z_rows_dev, mask_rows_dev, params, H: int, dtype: str, d: int = 32,
                 device="cuda"):
        torch = _torch()
        self.I = z_full_dev.shape[0]
        self.R, _, self.c = z_rows_dev.shape
        self.H, self.d, self.dtype = H, d, dtype
        self.z_full = z_full_dev
        self.z_rows = z_rows_dev
        self.mask = mask_rows_dev
        nbytes = lib.pairattn_rows_workspace_bytes(self.R, self.I, self.c, H, d, dtype_code(dtype))
        self.params = make_params(params, dtype, nbytes, device)
        self.bias = torch.empty((H, self.I, self.I), dtype=torch.float32, device=device)
        self.out = torch.empty_like(self.z_rows)

    def compute_bias(self, stream=None):
        lib.pairattn_tri_bias(self.z_full, self.params, self.bias, self.I, self.c, self.H, lib.PAIRATTN_START,
                              stream)
        return self.bias

    def rows(self, stream=None):
        lib.pairattn_tri_rows_fwd(self.z_rows, self.bias, self.mask, self.params, self.out, self.R, self.I, self.c,
                                  self.H, self.d, stream)
        return self.out

    def __call__(self, stream=None):
        self.compute_bias(stream)
        return self.rows(stream)
