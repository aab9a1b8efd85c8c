"""Python binding of the QSA C ABI (``include/qsa.h``): argument marshalling only.

Every step of the computation runs in the HIP library ``libqsa_amd.so``; this
module checks dtypes and shapes, allocates outputs and workspaces with torch,
passes raw device pointers and the current HIP stream, and turns status codes
into exceptions. It fails loudly when the library is missing: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa_amd.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "qsa.h")
TILE = 128
GROUP = 12
HEAD_DIM = 256

OK, ERR_NULL, ERR_SHAPE, ERR_HEADS, ERR_HEADDIM, ERR_SCALE, ERR_ALIGN, ERR_ROUTE_DTYPE, \
    ERR_WORKSPACE, ERR_DEVICE, ERR_LAUNCH = range(11)

_lib = None


class QSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"QSA status {status}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64),
                ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("D", ctypes.c_int64),
                ("W", ctypes.c_int64), ("route_is_i64", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


def library() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"QSA HIP library missing at {LIB_PATH}; "
                               "run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        P, S, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Dims)
        for name in ("qsa_forward_workspace_bytes", "qsa_backward_workspace_bytes",
                     "qsa_preprocess_workspace_bytes"):
            getattr(lib, name).restype = S
            getattr(lib, name).argtypes = [D]
        lib.qsa_forward.restype = ctypes.c_int
        lib.qsa_forward.argtypes = [D, P, P, P, P, ctypes.c_float, P, P, P, P, S, P]
        lib.qsa_backward.restype = ctypes.c_int
        lib.qsa_backward.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, S, P]
        lib.qsa_preprocess.restype = ctypes.c_int
        lib.qsa_preprocess.argtypes = [D] + [P] * 15 + [S, P]
        lib.qsa_status_string.restype = ctypes.c_char_p
        lib.qsa_status_string.argtypes = [ctypes.c_int]
        lib.qsa_version.restype = ctypes.c_int32
        lib.qsa_version.argtypes = []
        _lib = lib
    return _lib


def _raise(status: int) -> None:
    if status == OK:
        return
    msg = library().qsa_status_string(status).decode()
    if status in (ERR_SHAPE, ERR_HEADS, ERR_HEADDIM, ERR_SCALE, ERR_NULL, ERR_ALIGN):
        raise ValueError(f"QSA status {status}: {msg}")
    if status == ERR_ROUTE_DTYPE:
        raise TypeError(f"QSA status {status}: {msg}")
    raise QSAError(status, msg)


FLAG_DETERMINISTIC = 1  # QSA_FLAG_DETERMINISTIC


def make_dims(B, Sq, Skv, Hq, Hkv, D, W, route_is_i64=False, deterministic=False) -> Dims:
    return Dims(B, Sq, Skv, Hq, Hkv, D, W, 1 if route_is_i64 else 0,
                FLAG_DETERMINISTIC if deterministic else 0)


def _dims(q: torch.Tensor, k: torch.Tensor, routes: torch.Tensor, deterministic=False) -> Dims:
    if q.dim() != 4 or k.dim() != 4 or routes.dim() != 3:
        raise ValueError("q, k must be [B, S, H, 256] and routes [B, Sq, W]")
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != D or routes.shape[0] != B or routes.shape[1] != Sq:
        raise ValueError("inconsistent shapes")
    if routes.dtype not in (torch.int32, torch.int64):
        raise TypeError("routes must be int32 or int64")
    return make_dims(B, Sq, Skv, Hq, Hkv, D, routes.shape[2], routes.dtype == torch.int64,
                     deterministic)


def _check(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    return t.contiguous()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def forward_workspace_bytes(dims: Dims) -> int:
    return int(library().qsa_forward_workspace_bytes(ctypes.byref(dims)))


def backward_workspace_bytes(dims: Dims) -> int:
    return int(library().qsa_backward_workspace_bytes(ctypes.byref(dims)))


def preprocess_workspace_bytes(dims: Dims) -> int:
    return int(library().qsa_preprocess_workspace_bytes(ctypes.byref(dims)))


def forward(q, k, v, routes, scale: Optional[float] = None, *, out=None, out_fp32=None, lse=None,
            workspace=None, deterministic: bool = False):
    """QSA forward. Returns ``(out bf16, out_fp32, lse [B, Hq, Sq])``.

    ``deterministic`` sets QSA_FLAG_DETERMINISTIC (bitwise reproducible)."""
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    routes = routes.contiguous()
    if not routes.is_cuda:
        raise ValueError("routes must be a GPU tensor")
    dims = _dims(q, k, routes, deterministic)
    if v.shape != k.shape:
        raise ValueError("v must have k's shape")
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    B, Sq, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if out_fp32 is None:
        out_fp32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    lib = library()
    need = lib.qsa_forward_workspace_bytes(ctypes.byref(dims))
    if need == 0:
        _raise(lib.qsa_forward(ctypes.byref(dims), None, None, None, None, float(scale), None,
                               None, None, None, 0, None) or ERR_SHAPE)
    ws = _workspace(need, q.device, workspace)
    st = lib.qsa_forward(ctypes.byref(dims), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         routes.data_ptr(), float(scale), out.data_ptr(), out_fp32.data_ptr(),
                         lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                         _stream())
    _raise(st)
    return out, out_fp32, lse


def backward(grad_out, q, k, v, out_fp32, lse, routes, scale: Optional[float] = None, *,
             dq=None, dk=None, dv=None, workspace=None, deterministic: bool = False):
    """QSA backward. Returns ``(dq, dk, dv)`` in bf16.

    ``deterministic`` sets QSA_FLAG_DETERMINISTIC (bitwise reproducible)."""
    grad_out = _check(grad_out, torch.bfloat16, "grad_out")
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    out_fp32 = _check(out_fp32, torch.float32, "out_fp32")
    lse = _check(lse, torch.float32, "lse")
    routes = routes.contiguous()
    dims = _dims(q, k, routes, deterministic)
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    if grad_out.shape != q.shape or out_fp32.shape != q.shape:
        raise ValueError("grad_out and out_fp32 must have q's shape")
    if lse.shape != (q.shape[0], q.shape[2], q.shape[1]):
        raise ValueError("lse must be [B, Hq, Sq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = library()
    need = lib.qsa_backward_workspace_bytes(ctypes.byref(dims))
    if need == 0:
        _raise(lib.qsa_backward(ctypes.byref(dims), *([None] * 7), float(scale), None, None,
                                None, None, 0, None) or ERR_SHAPE)
    ws = _workspace(need, q.device, workspace)
    st = lib.qsa_backward(ctypes.byref(dims), grad_out.data_ptr(), q.data_ptr(), k.data_ptr(),
                          v.data_ptr(), out_fp32.data_ptr(), lse.data_ptr(), routes.data_ptr(),
                          float(scale), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    _raise(st)
    return dq, dk, dv


def preprocess(routes: torch.Tensor, Skv: int, *, with_row_keys: bool = True) -> dict:
    """Run the route preprocessing alone; returns its tables as GPU tensors."""
    routes = routes.contiguous()
    if not routes.is_cuda:
        raise ValueError("routes must be a GPU tensor")
    if routes.dtype not in (torch.int32, torch.int64):
        raise TypeError("routes must be int32 or int64")
    B, Sq, W = routes.shape
    dims = make_dims(B, Sq, Skv, GROUP, 1, HEAD_DIM, W, routes.dtype == torch.int64)
    nqt, nkt = -(-Sq // TILE), -(-Skv // TILE)
    dev = routes.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = {
        "memb": torch.empty((B, Sq, nkt * TILE), dtype=torch.uint8, device=dev),
        "has_routes": torch.empty((B, Sq), dtype=torch.uint8, device=dev),
        "kinds": torch.empty((B, nqt, nkt), **i32),
        "fwd_p_cnt": torch.empty((B, nqt), **i32), "fwd_p_idx": torch.empty((B, nqt, nkt), **i32),
        "fwd_f_cnt": torch.empty((B, nqt), **i32), "fwd_f_idx": torch.empty((B, nqt, nkt), **i32),
        "rev_p_cnt": torch.empty((B, nkt), **i32), "rev_p_idx": torch.empty((B, nkt, nqt), **i32),
        "rev_f_cnt": torch.empty((B, nkt), **i32), "rev_f_idx": torch.empty((B, nkt, nqt), **i32),
    }
    if with_row_keys:
        out["row_keys"] = torch.empty((B, Sq, W), **i32)
        out["row_cnt"] = torch.empty((B, Sq), **i32)
    lib = library()
    need = lib.qsa_preprocess_workspace_bytes(ctypes.byref(dims))
    if need == 0:
        _raise(ERR_SHAPE)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    order = ["memb", "has_routes", "kinds", "fwd_p_cnt", "fwd_p_idx", "fwd_f_cnt", "fwd_f_idx",
             "rev_p_cnt", "rev_p_idx", "rev_f_cnt", "rev_f_idx"]
    st = lib.qsa_preprocess(ctypes.byref(dims), routes.data_ptr(),
                            *[out[n].data_ptr() for n in order],
                            _ptr(out.get("row_keys")), _ptr(out.get("row_cnt")),
                            ws.data_ptr(), need, _stream())
    _raise(st)
    return out
