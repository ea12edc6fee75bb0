"""ctypes binding of libpairattn.so (the C ABI in include/pairattn.h).

Argument marshalling only: every function forwards to the entry point of
the same name.  Tensors may be torch tensors (their device pointer is
passed), raw integer addresses, or None (NULL).  PyTorch is used for device
memory and streams; no computation happens here.

The shared library is loaded on first use from this package directory (or
from the path in PAIRATTN_LIB, e.g. the host-sanitized build) and a missing
library raises ``PairAttnLibraryMissing``: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpairattn.so")
# the same library with the kernels' index checks on (pairattn_debug_status)
DEBUG_LIB_PATH = os.path.join(PKG_DIR, "libpairattn_debug.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "pairattn.h")

PAIRATTN_OK = 0
PAIRATTN_ERR_ARG = 1
PAIRATTN_ERR_UNSUPPORTED = 2
PAIRATTN_ERR_WORKSPACE = 3
PAIRATTN_ERR_DEVICE = 4
PAIRATTN_ERR_HIP = 5

# size of the static scratch of pairattn_tri_fwd_noalloc (PAIRATTN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20

# bits of pairattn_tri_partial_fwd's accumulate argument
PAIRATTN_PARTIAL_MERGE = 1
PAIRATTN_PARTIAL_Q_READY = 2
PAIRATTN_START = 0
PAIRATTN_END = 1
PAIRATTN_F32 = 0
PAIRATTN_BF16 = 1


class PairAttnLibraryMissing(RuntimeError):
    pass


class PairAttnError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed with status {status} ({status_string(status)}): {detail}")


class pairattn_params(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("ln_gamma", ctypes.c_void_p),
        ("ln_beta", ctypes.c_void_p),
        ("w_q", ctypes.c_void_p),
        ("w_k", ctypes.c_void_p),
        ("w_v", ctypes.c_void_p),
        ("w_g", ctypes.c_void_p),
        ("b_g", ctypes.c_void_p),
        ("w_b", ctypes.c_void_p),
        ("w_o", ctypes.c_void_p),
        ("b_o", ctypes.c_void_p),
        ("lnz_gamma", ctypes.c_void_p),
        ("lnz_beta", ctypes.c_void_p),
        ("ln_eps", ctypes.c_float),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None

_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_P = ctypes.c_void_p
_PP = ctypes.POINTER(pairattn_params)

_SIGNATURES = {
    "pairattn_tri_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I32]),
    "pairattn_msa_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I64, _I64, _I32]),
    "pairattn_rows_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I64, _I32]),
    "pairattn_tri_fwd": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I32, _P]),
    "pairattn_tri_fwd_noalloc": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I32, _P]),
    "pairattn_msa_row_fwd": (ctypes.c_int, [_P, _P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
    "pairattn_tri_bias": (ctypes.c_int, [_P, _PP, _P, _I64, _I64, _I64, _I32, _P]),
    "pairattn_tri_rows_fwd": (ctypes.c_int, [_P, _P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    "pairattn_tri_chunked_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I32, _I64]),
    "pairattn_tri_chunked_fwd": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I32, _I64, _P]),
    "pairattn_validate_tri_chunked": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I32, _I64]),
    "pairattn_tri_partial_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I64, _I64, _I32]),
    "pairattn_tri_partial_fwd": (ctypes.c_int, [_P, _P, _P, _P, _PP, _P, _P, _I32, _I64, _I64, _I64, _I64, _I64, _I64,
                                                _P]),
    "pairattn_tri_partial_finish_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I64, _I32]),
    "pairattn_tri_partial_finish": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I64, _P]),
    "pairattn_validate_tri_partial": (ctypes.c_int, [_P, _P, _P, _P, _PP, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                                     _I64]),
    "pairattn_validate_tri_partial_finish": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I64]),
    "pairattn_validate_tri": (ctypes.c_int, [_P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I32]),
    "pairattn_validate_msa": (ctypes.c_int, [_P, _P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I64, _I64]),
    "pairattn_validate_rows": (ctypes.c_int, [_P, _P, _P, _PP, _P, _I64, _I64, _I64, _I64, _I64]),
    "pairattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pairattn_last_error": (ctypes.c_char_p, []),
    "pairattn_version": (ctypes.c_int, []),
    "pairattn_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "pairattn_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p),
                                            ctypes.c_int]),
    "pairattn_calibrate_exp2": (ctypes.c_int, [_P, _I64, _P]),
    "pairattn_debug_status": (ctypes.c_int, [_P, _P]),
}


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and return the shared library."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("PAIRATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise PairAttnLibraryMissing(
            f"{path} not found: build it with `python -m pair_representation_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions declared in include/pairattn.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pairattn_[a-z_]+)\s*\(", text)))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)!r} as a device pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except Exception:  # pragma: no cover - torch missing
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_string(status: int) -> str:
    return load().pairattn_status_string(status).decode()


def last_error() -> str:
    return load().pairattn_last_error().decode()


def _check(status: int, func: str) -> int:
    if status != PAIRATTN_OK:
        raise PairAttnError(status, func, last_error())
    return status


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def pairattn_tri_workspace_bytes(I, c_z, H, d, dtype) -> int:
    return load().pairattn_tri_workspace_bytes(I, c_z, H, d, dtype)


def pairattn_msa_workspace_bytes(S, I, c_m, c_z, H, d, dtype) -> int:
    return load().pairattn_msa_workspace_bytes(S, I, c_m, c_z, H, d, dtype)


def pairattn_rows_workspace_bytes(R, I, c_z, H, d, dtype) -> int:
    return load().pairattn_rows_workspace_bytes(R, I, c_z, H, d, dtype)


def pairattn_tri_fwd(z, mask, params, out, I, c_z, H, d, orientation, stream=None, check=True) -> int:
    st = load().pairattn_tri_fwd(_ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), I, c_z, H, d,
                                 orientation, _stream(stream))
    return _check(st, "pairattn_tri_fwd") if check else st


def pairattn_tri_fwd_noalloc(z, mask, params, out, I, c_z, H, d, orientation, stream=None, check=True) -> int:
    st = load().pairattn_tri_fwd_noalloc(_ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), I, c_z, H,
                                         d, orientation, _stream(stream))
    return _check(st, "pairattn_tri_fwd_noalloc") if check else st


def pairattn_msa_row_fwd(m, z, mask, params, out, S, I, c_m, c_z, H, d, stream=None, check=True) -> int:
    st = load().pairattn_msa_row_fwd(_ptr(m), _ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), S, I,
                                     c_m, c_z, H, d, _stream(stream))
    return _check(st, "pairattn_msa_row_fwd") if check else st


def pairattn_tri_bias(z, params, bias, I, c_z, H, orientation, stream=None, check=True) -> int:
    st = load().pairattn_tri_bias(_ptr(z), ctypes.byref(params.struct()), _ptr(bias), I, c_z, H, orientation,
                                  _stream(stream))
    return _check(st, "pairattn_tri_bias") if check else st


def pairattn_tri_rows_fwd(z_rows, bias, mask_rows, params, out_rows, R, I, c_z, H, d, stream=None,
                          check=True) -> int:
    st = load().pairattn_tri_rows_fwd(_ptr(z_rows), _ptr(bias), _ptr(mask_rows), ctypes.byref(params.struct()),
                                      _ptr(out_rows), R, I, c_z, H, d, _stream(stream))
    return _check(st, "pairattn_tri_rows_fwd") if check else st


def pairattn_tri_chunked_workspace_bytes(I, c_z, H, d, dtype, block) -> int:
    return load().pairattn_tri_chunked_workspace_bytes(I, c_z, H, d, dtype, block)


def pairattn_tri_chunked_fwd(z, mask, params, out, I, c_z, H, d, orientation, block, stream=None,
                             check=True) -> int:
    st = load().pairattn_tri_chunked_fwd(_ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), I, c_z, H,
                                         d, orientation, block, _stream(stream))
    return _check(st, "pairattn_tri_chunked_fwd") if check else st


def pairattn_validate_tri_chunked(z, mask, params, out, I, c_z, H, d, orientation, block) -> int:
    return load().pairattn_validate_tri_chunked(_ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), I,
                                                c_z, H, d, orientation, block)


def pairattn_tri_partial_workspace_bytes(R, Jq, Kn, c_z, H, d, dtype) -> int:
    return load().pairattn_tri_partial_workspace_bytes(R, Jq, Kn, c_z, H, d, dtype)


def pairattn_tri_partial_fwd(q_pairs, kv_pairs, bias, mask, params, o, lse, accumulate, R, Jq, Kn, c_z, H, d,
                             stream=None, check=True) -> int:
    st = load().pairattn_tri_partial_fwd(_ptr(q_pairs), _ptr(kv_pairs), _ptr(bias), _ptr(mask),
                                         ctypes.byref(params.struct()), _ptr(o), _ptr(lse), int(accumulate),
                                         R, Jq, Kn, c_z, H, d, _stream(stream))
    return _check(st, "pairattn_tri_partial_fwd") if check else st


def pairattn_tri_partial_finish_workspace_bytes(R, Jq, c_z, H, d, dtype) -> int:
    return load().pairattn_tri_partial_finish_workspace_bytes(R, Jq, c_z, H, d, dtype)


def pairattn_tri_partial_finish(q_pairs, o, params, out, R, Jq, c_z, H, d, stream=None, check=True) -> int:
    st = load().pairattn_tri_partial_finish(_ptr(q_pairs), _ptr(o), ctypes.byref(params.struct()), _ptr(out), R, Jq,
                                            c_z, H, d, _stream(stream))
    return _check(st, "pairattn_tri_partial_finish") if check else st


def pairattn_validate_tri_partial(q_pairs, kv_pairs, bias, mask, params, o, lse, R, Jq, Kn, c_z, H, d) -> int:
    return load().pairattn_validate_tri_partial(_ptr(q_pairs), _ptr(kv_pairs), _ptr(bias), _ptr(mask),
                                                ctypes.byref(params.struct()), _ptr(o), _ptr(lse), R, Jq, Kn, c_z,
                                                H, d)


def pairattn_validate_tri_partial_finish(q_pairs, o, params, out, R, Jq, c_z, H, d) -> int:
    return load().pairattn_validate_tri_partial_finish(_ptr(q_pairs), _ptr(o), ctypes.byref(params.struct()),
                                                       _ptr(out), R, Jq, c_z, H, d)


def pairattn_validate_tri(z, mask, params, out, I, c_z, H, d, orientation) -> int:
    return load().pairattn_validate_tri(_ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), I, c_z, H,
                                        d, orientation)


def pairattn_validate_msa(m, z, mask, params, out, S, I, c_m, c_z, H, d) -> int:
    return load().pairattn_validate_msa(_ptr(m), _ptr(z), _ptr(mask), ctypes.byref(params.struct()), _ptr(out), S,
                                        I, c_m, c_z, H, d)


def pairattn_validate_rows(z_rows, bias, mask_rows, params, out_rows, R, I, c_z, H, d) -> int:
    return load().pairattn_validate_rows(_ptr(z_rows), _ptr(bias), _ptr(mask_rows), ctypes.byref(params.struct()),
                                         _ptr(out_rows), R, I, c_z, H, d)


def pairattn_timing_enable(enable: bool) -> bool:
    st = load().pairattn_timing_enable(1 if enable else 0)
    if st < 0:
        raise PairAttnError(-st, "pairattn_timing_enable", last_error())
    return bool(st)


def pairattn_debug_status():
    """(flags, checking) of the debug build's index checks (flags cleared);
    (0, 0) from the release build."""
    f = ctypes.c_uint32(0)
    c = ctypes.c_int32(0)
    _check(load().pairattn_debug_status(ctypes.byref(f), ctypes.byref(c)), "pairattn_debug_status")
    return int(f.value), int(c.value)


def pairattn_calibrate_exp2(out, iters: int, stream=None, check=True) -> int:
    st = load().pairattn_calibrate_exp2(_ptr(out), iters, _stream(stream))
    return _check(st, "pairattn_calibrate_exp2") if check else st


def pairattn_timing_read(cap: int = 1024) -> list:
    """[(stage name, ms), ...] of every call on this thread since the last
    read, in launch order (waits for the last one)."""
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    n = load().pairattn_timing_read(ms, names, cap)
    if n < 0:
        raise PairAttnError(-n, "pairattn_timing_read", last_error())
    return [(names[i].decode(), float(ms[i])) for i in range(n)]


# ----------------------------------------------------------------------------
# parameter holder
# ----------------------------------------------------------------------------
class Params:
    """Keeps the weight tensors (and the workspace) alive and builds the
    ``pairattn_params`` struct that the entry points read."""

    NAMES = ("ln_gamma", "ln_beta", "w_q", "w_k", "w_v", "w_g", "b_g", "w_b", "w_o", "b_o",
             "lnz_gamma", "lnz_beta")

    def __init__(self, dtype: int, eps: float = 1e-5, workspace=None, workspace_bytes: Optional[int] = None,
                 **tensors):
        self.dtype = dtype
        self.eps = eps
        self.tensors = {k: tensors.get(k) for k in self.NAMES}
        unknown = set(tensors) - set(self.NAMES)
        if unknown:
            raise TypeError(f"unknown parameter names {sorted(unknown)}")
        self.workspace = workspace
        self.workspace_bytes = workspace_bytes

    def struct(self) -> pairattn_params:
        s = pairattn_params()
        s.dtype = self.dtype
        for k in self.NAMES:
            setattr(s, k, _ptr(self.tensors[k]))
        s.ln_eps = float(self.eps)
        s.workspace = _ptr(self.workspace)
        if self.workspace_bytes is not None:
            s.workspace_bytes = int(self.workspace_bytes)
        elif self.workspace is not None and hasattr(self.workspace, "numel"):
            s.workspace_bytes = self.workspace.numel() * self.workspace.element_size()
        else:
            s.workspace_bytes = 0
        return s
