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
    ERR_WORKSPACE, ERR_DEVICE, ERR_LAUNCH, ERR_SCRATCH, ERR_PLAN = range(13)
PLAN_TAG = 0x51534150  # QSA_PLAN_TAG
NOALLOC_SCRATCH_BYTES = 64 << 20  # QSA_NOALLOC_SCRATCH_BYTES

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


class BlockDims(ctypes.Structure):
    """``qsa_block_dims``: packed tokens T, blocks NB, heads, block size, flags."""
    _fields_ = [("T", ctypes.c_int64), ("NB", ctypes.c_int64), ("Hq", ctypes.c_int64),
                ("Hkv", ctypes.c_int64), ("D", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class DocDims(ctypes.Structure):
    """``qsa_doc_dims``: shapes, the query shard's global start, flags."""
    _fields_ = [("B", ctypes.c_int64), ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64),
                ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("D", ctypes.c_int64),
                ("q_global_start", ctypes.c_int64), ("flags", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class SelectDims(ctypes.Structure):
    """``qsa_select_dims``: selector shapes, the query shard's position, top_k."""
    _fields_ = [("B", ctypes.c_int64), ("Sq", ctypes.c_int64), ("NB", ctypes.c_int64),
                ("q_offset", ctypes.c_int64), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("flags", ctypes.c_int32)]


class PlanStruct(ctypes.Structure):
    """``qsa_plan``: the host record of a built route plan."""
    _fields_ = [("dims", Dims), ("mem", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
                ("device", ctypes.c_int32), ("tag", ctypes.c_uint32)]


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
                     "qsa_preprocess_workspace_bytes", "qsa_plan_bytes",
                     "qsa_forward_planned_workspace_bytes",
                     "qsa_backward_planned_workspace_bytes"):
            getattr(lib, name).restype = S
            getattr(lib, name).argtypes = [D]
        lib.qsa_forward.restype = ctypes.c_int
        lib.qsa_forward.argtypes = [D, P, P, P, P, ctypes.c_float, P, P, P, P, S, P]
        lib.qsa_forward_noalloc.restype = ctypes.c_int
        lib.qsa_forward_noalloc.argtypes = [D, P, P, P, P, ctypes.c_float, P, P, P, P]
        lib.qsa_backward.restype = ctypes.c_int
        lib.qsa_backward.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, S, P]
        lib.qsa_preprocess.restype = ctypes.c_int
        lib.qsa_preprocess.argtypes = [D] + [P] * 15 + [S, P]
        PL = ctypes.POINTER(PlanStruct)
        lib.qsa_plan_build.restype = ctypes.c_int
        lib.qsa_plan_build.argtypes = [D, P, P, S, PL, P]
        lib.qsa_forward_planned.restype = ctypes.c_int
        lib.qsa_forward_planned.argtypes = [PL, P, P, P, ctypes.c_float, P, P, P, P, S, P]
        lib.qsa_backward_planned.restype = ctypes.c_int
        lib.qsa_backward_planned.argtypes = [PL, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, S,
                                             P]
        BD = ctypes.POINTER(BlockDims)
        for name in ("qsa_block_plan_bytes", "qsa_block_forward_workspace_bytes",
                     "qsa_block_backward_workspace_bytes"):
            getattr(lib, name).restype = S
            getattr(lib, name).argtypes = [BD]
        lib.qsa_block_plan_build.restype = ctypes.c_int
        lib.qsa_block_plan_build.argtypes = [BD] + [P] * 7 + [P, S, PL, P]
        lib.qsa_block_forward.restype = ctypes.c_int
        lib.qsa_block_forward.argtypes = [BD] + [P] * 10 + [ctypes.c_float] + [P] * 4 + [S, P]
        lib.qsa_block_backward.restype = ctypes.c_int
        lib.qsa_block_backward.argtypes = [BD] + [P] * 13 + [ctypes.c_float] + [P] * 4 + [S, P]
        DD = ctypes.POINTER(DocDims)
        for name in ("qsa_doc_plan_bytes", "qsa_doc_forward_workspace_bytes",
                     "qsa_doc_backward_workspace_bytes"):
            getattr(lib, name).restype = S
            getattr(lib, name).argtypes = [DD]
        lib.qsa_doc_plan_build.restype = ctypes.c_int
        lib.qsa_doc_plan_build.argtypes = [DD, P, P, P, S, PL, P]
        lib.qsa_doc_forward.restype = ctypes.c_int
        lib.qsa_doc_forward.argtypes = [DD] + [P] * 5 + [ctypes.c_float] + [P] * 4 + [S, P]
        lib.qsa_doc_backward.restype = ctypes.c_int
        lib.qsa_doc_backward.argtypes = [DD] + [P] * 8 + [ctypes.c_float] + [P] * 4 + [S, P]
        SD = ctypes.POINTER(SelectDims)
        lib.qsa_select_workspace_bytes.restype = S
        lib.qsa_select_workspace_bytes.argtypes = [SD]
        lib.qsa_select.restype = ctypes.c_int
        lib.qsa_select.argtypes = [SD, P, P, P, P, ctypes.c_float, P, P, P, P, S, P]
        lib.qsa_plan_tables.restype = ctypes.c_int
        lib.qsa_plan_tables.argtypes = [PL] + [P] * 12 + [P]
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
    if status in (ERR_SHAPE, ERR_HEADS, ERR_HEADDIM, ERR_SCALE, ERR_NULL, ERR_ALIGN,
                  ERR_SCRATCH, ERR_PLAN):
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


def forward_noalloc(q, k, v, routes, scale: Optional[float] = None, *, out, out_fp32, lse,
                    deterministic: bool = False):
    """QSA forward through ``qsa_forward_noalloc``: the caller passes every output,
    and the library uses its fixed device scratch as workspace (no allocation)."""
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    if not routes.is_cuda:
        raise ValueError("routes must be a GPU tensor")
    for t, name in ((routes, "routes"), (out, "out"), (out_fp32, "out_fp32"), (lse, "lse")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dims = _dims(q, k, routes, deterministic)
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    st = library().qsa_forward_noalloc(ctypes.byref(dims), q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), routes.data_ptr(), float(scale),
                                       out.data_ptr(), out_fp32.data_ptr(), lse.data_ptr(),
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


class Plan:
    """A built route plan: the ``qsa_plan`` record and the device buffer it names.

    Keep the object alive while planned calls may still run on the stream: it
    owns the buffer."""

    def __init__(self, struct: PlanStruct, mem: torch.Tensor):
        self.struct = struct
        self.mem = mem

    @property
    def dims(self) -> Dims:
        return self.struct.dims


def plan_bytes(dims: Dims) -> int:
    return int(library().qsa_plan_bytes(ctypes.byref(dims)))


def plan_build(routes: torch.Tensor, Skv: int, *, Hkv: int = 1, deterministic: bool = False,
               plan_mem: Optional[torch.Tensor] = None) -> Plan:
    """Build the route plan of ``routes`` [B, Sq, W] for ``Skv`` keys and ``Hkv`` KV heads
    (``qsa_plan_build``); forward_planned and backward_planned reuse it."""
    routes = routes.contiguous()
    if not routes.is_cuda:
        raise ValueError("routes must be a GPU tensor")
    if routes.dtype not in (torch.int32, torch.int64):
        raise TypeError("routes must be int32 or int64")
    if routes.dim() != 3:
        raise ValueError("routes must be [B, Sq, W]")
    B, Sq, W = routes.shape
    dims = make_dims(B, Sq, Skv, GROUP * Hkv, Hkv, HEAD_DIM, W, routes.dtype == torch.int64,
                     deterministic)
    lib = library()
    need = lib.qsa_plan_bytes(ctypes.byref(dims))
    mem = _workspace(need, routes.device, plan_mem)
    struct = PlanStruct()
    st = lib.qsa_plan_build(ctypes.byref(dims), routes.data_ptr(), mem.data_ptr(),
                            mem.numel() * mem.element_size(), ctypes.byref(struct), _stream())
    _raise(st)
    return Plan(struct, mem)


def _plan_shapes(plan: Plan):
    d = plan.dims
    return (d.B, d.Sq, d.Hq, d.D), (d.B, d.Skv, d.Hkv, d.D), (d.B, d.Hq, d.Sq)


def forward_planned(plan: Plan, q, k, v, scale: Optional[float] = None, *, out=None,
                    out_fp32=None, lse=None, workspace=None):
    """QSA forward on a built plan (``qsa_forward_planned``): no route preprocessing."""
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    qs, ks, ls = _plan_shapes(plan)
    if tuple(q.shape) != qs or tuple(k.shape) != ks or tuple(v.shape) != ks:
        raise ValueError(f"q must be {qs} and k, v {ks} for this plan")
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    out = torch.empty_like(q) if out is None else out
    out_fp32 = torch.empty(qs, dtype=torch.float32, device=q.device) if out_fp32 is None \
        else out_fp32
    lse = torch.empty(ls, dtype=torch.float32, device=q.device) if lse is None else lse
    lib = library()
    need = lib.qsa_forward_planned_workspace_bytes(ctypes.byref(plan.dims))
    ws = _workspace(need, q.device, workspace)
    st = lib.qsa_forward_planned(ctypes.byref(plan.struct), q.data_ptr(), k.data_ptr(),
                                 v.data_ptr(), float(scale), out.data_ptr(), out_fp32.data_ptr(),
                                 lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream())
    _raise(st)
    return out, out_fp32, lse


def backward_planned(plan: Plan, grad_out, q, k, v, out_fp32, lse, scale: Optional[float] = None,
                     *, dq=None, dk=None, dv=None, workspace=None):
    """QSA backward on a built plan (``qsa_backward_planned``): no route preprocessing."""
    grad_out = _check(grad_out, torch.bfloat16, "grad_out")
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    out_fp32 = _check(out_fp32, torch.float32, "out_fp32")
    lse = _check(lse, torch.float32, "lse")
    qs, ks, ls = _plan_shapes(plan)
    if tuple(q.shape) != qs or tuple(grad_out.shape) != qs or tuple(out_fp32.shape) != qs:
        raise ValueError(f"q, grad_out and out_fp32 must be {qs} for this plan")
    if tuple(k.shape) != ks or tuple(v.shape) != ks:
        raise ValueError(f"k and v must be {ks} for this plan")
    if tuple(lse.shape) != ls:
        raise ValueError(f"lse must be {ls} for this plan")
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = library()
    need = lib.qsa_backward_planned_workspace_bytes(ctypes.byref(plan.dims))
    ws = _workspace(need, q.device, workspace)
    st = lib.qsa_backward_planned(ctypes.byref(plan.struct), grad_out.data_ptr(), q.data_ptr(),
                                  k.data_ptr(), v.data_ptr(), out_fp32.data_ptr(),
                                  lse.data_ptr(), float(scale), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                  _stream())
    _raise(st)
    return dq, dk, dv


def plan_tables(plan: Plan) -> dict:
    """Copies of a plan's tables (``qsa_plan_tables``) as GPU tensors."""
    d = plan.dims
    nqt, nkt = -(-d.Sq // TILE), -(-d.Skv // TILE)
    dev = plan.mem.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = {
        "mbits": torch.empty((d.B, d.Sq, nkt * TILE // 32), **i32),
        "kinds": torch.empty((d.B, nqt, nkt), **i32),
        "fwd_p_cnt": torch.empty((d.B, nqt), **i32), "fwd_p_idx": torch.empty((d.B, nqt, nkt), **i32),
        "fwd_f_cnt": torch.empty((d.B, nqt), **i32), "fwd_f_idx": torch.empty((d.B, nqt, nkt), **i32),
        "rev_p_cnt": torch.empty((d.B, nkt), **i32), "rev_p_idx": torch.empty((d.B, nkt, nqt), **i32),
        "rev_f_cnt": torch.empty((d.B, nkt), **i32), "rev_f_idx": torch.empty((d.B, nkt, nqt), **i32),
        "row_keys": torch.empty((d.B, d.Sq, d.W), **i32),
        "row_cnt": torch.empty((d.B, d.Sq), **i32),
    }
    st = library().qsa_plan_tables(ctypes.byref(plan.struct), *[t.data_ptr() for t in out.values()],
                                   _stream())
    _raise(st)
    return out


def _block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last):
    sel = _check(sel_blocks, torch.uint8, "sel_blocks")
    meta = [_check(t, torch.int32, n) for t, n in ((lo, "lo"), (hi, "hi"), (blk_base, "blk_base"),
                                                  (tok_base, "tok_base"))]
    spans = [_check(t, torch.int32, n) for t, n in ((block_first, "block_first"),
                                                   (block_last, "block_last"))]
    if sel.dim() != 2:
        raise ValueError("sel_blocks must be [T, NB]")
    T, NB = sel.shape
    if any(tuple(t.shape) != (T,) for t in meta) or any(tuple(t.shape) != (NB,) for t in spans):
        raise ValueError("lo, hi, blk_base, tok_base must be [T] and block_first, block_last [NB]")
    return sel, meta, spans


def block_dims(T: int, NB: int, Hkv: int = 1, block_size: int = 4,
               deterministic: bool = False) -> BlockDims:
    return BlockDims(T, NB, GROUP * Hkv, Hkv, HEAD_DIM, block_size,
                     FLAG_DETERMINISTIC if deterministic else 0)


def block_plan_build(sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last, *,
                     Hkv: int = 1, block_size: int = 4, deterministic: bool = False,
                     plan_mem: Optional[torch.Tensor] = None) -> Plan:
    """Build a route plan from a block-selection bitmap (``qsa_block_plan_build``)."""
    sel, meta, spans = _block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first,
                                   block_last)
    bd = block_dims(sel.shape[0], sel.shape[1], Hkv, block_size, deterministic)
    lib = library()
    need = lib.qsa_block_plan_bytes(ctypes.byref(bd))
    mem = _workspace(need, sel.device, plan_mem)
    struct = PlanStruct()
    st = lib.qsa_block_plan_build(ctypes.byref(bd), sel.data_ptr(),
                                  *[t.data_ptr() for t in meta + spans], mem.data_ptr(),
                                  mem.numel() * mem.element_size(), ctypes.byref(struct),
                                  _stream())
    _raise(st)
    return Plan(struct, mem)


def block_forward(q, k, v, sel_blocks, lo, hi, blk_base, tok_base, block_first, block_last,
                  scale: Optional[float] = None, *, block_size: int = 4, out=None, out_fp32=None,
                  lse=None, workspace=None, deterministic: bool = False):
    """QSA forward on packed tokens with a block-selection bitmap (``qsa_block_forward``).
    q [T, Hq, 256], k, v [T, Hkv, 256]; returns ``(out, out_fp32, lse [Hq, T])``."""
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    sel, meta, spans = _block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first,
                                   block_last)
    T, NB = sel.shape
    if q.dim() != 3 or q.shape[0] != T or k.shape != v.shape or k.dim() != 3 or k.shape[0] != T:
        raise ValueError("q must be [T, Hq, 256] and k, v [T, Hkv, 256]")
    Hq, Hkv = q.shape[1], k.shape[1]
    bd = BlockDims(T, NB, Hq, Hkv, q.shape[2], block_size, FLAG_DETERMINISTIC if deterministic
                   else 0)
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    out = torch.empty_like(q) if out is None else out
    out_fp32 = torch.empty(q.shape, dtype=torch.float32, device=q.device) if out_fp32 is None \
        else out_fp32
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    lib = library()
    ws = _workspace(lib.qsa_block_forward_workspace_bytes(ctypes.byref(bd)), q.device, workspace)
    st = lib.qsa_block_forward(ctypes.byref(bd), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               sel.data_ptr(), *[t.data_ptr() for t in meta + spans],
                               float(scale), out.data_ptr(), out_fp32.data_ptr(), lse.data_ptr(),
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    _raise(st)
    return out, out_fp32, lse


def block_backward(grad_out, q, k, v, out_fp32, lse, sel_blocks, lo, hi, blk_base, tok_base,
                   block_first, block_last, scale: Optional[float] = None, *,
                   block_size: int = 4, dq=None, dk=None, dv=None, workspace=None,
                   deterministic: bool = False):
    """QSA backward on packed tokens with a block-selection bitmap (``qsa_block_backward``).
    Returns ``(dq, dk, dv)``."""
    grad_out = _check(grad_out, torch.bfloat16, "grad_out")
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    out_fp32 = _check(out_fp32, torch.float32, "out_fp32")
    lse = _check(lse, torch.float32, "lse")
    sel, meta, spans = _block_meta(sel_blocks, lo, hi, blk_base, tok_base, block_first,
                                   block_last)
    T, NB = sel.shape
    if q.dim() != 3 or q.shape[0] != T or k.shape != v.shape or k.dim() != 3 or k.shape[0] != T:
        raise ValueError("q must be [T, Hq, 256] and k, v [T, Hkv, 256]")
    if grad_out.shape != q.shape or out_fp32.shape != q.shape:
        raise ValueError("grad_out and out_fp32 must have q's shape")
    Hq, Hkv = q.shape[1], k.shape[1]
    if tuple(lse.shape) != (Hq, T):
        raise ValueError("lse must be [Hq, T]")
    bd = BlockDims(T, NB, Hq, Hkv, q.shape[2], block_size, FLAG_DETERMINISTIC if deterministic
                   else 0)
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = library()
    ws = _workspace(lib.qsa_block_backward_workspace_bytes(ctypes.byref(bd)), q.device,
                    workspace)
    st = lib.qsa_block_backward(ctypes.byref(bd), grad_out.data_ptr(), q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), out_fp32.data_ptr(), lse.data_ptr(),
                                sel.data_ptr(), *[t.data_ptr() for t in meta + spans],
                                float(scale), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    _raise(st)
    return dq, dk, dv


def _doc_args(q, k, q_doc_ids, kv_doc_ids, q_global_start, deterministic):
    qd = _check(q_doc_ids, torch.int32, "q_doc_ids")
    kd = _check(kv_doc_ids, torch.int32, "kv_doc_ids")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Sq, Hq, 256] and k, v [B, Skv, Hkv, 256]")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(qd.shape) != (B, Sq) or tuple(kd.shape) != (B, Skv):
        raise ValueError("q_doc_ids must be [B, Sq] and kv_doc_ids [B, Skv]")
    dd = DocDims(B, Sq, Skv, Hq, Hkv, D, int(q_global_start),
                 FLAG_DETERMINISTIC if deterministic else 0, 0)
    return dd, qd, kd


def doc_plan_build(q_doc_ids, kv_doc_ids, *, Hkv: int = 1, q_global_start: int = 0,
                   deterministic: bool = False, plan_mem: Optional[torch.Tensor] = None) -> Plan:
    """Build a route plan of causal attention within documents (``qsa_doc_plan_build``):
    q_doc_ids [B, Sq], kv_doc_ids [B, Skv], 1-based, 0 = padding."""
    qd = _check(q_doc_ids, torch.int32, "q_doc_ids")
    kd = _check(kv_doc_ids, torch.int32, "kv_doc_ids")
    if qd.dim() != 2 or kd.dim() != 2 or qd.shape[0] != kd.shape[0]:
        raise ValueError("q_doc_ids must be [B, Sq] and kv_doc_ids [B, Skv]")
    dd = DocDims(qd.shape[0], qd.shape[1], kd.shape[1], GROUP * Hkv, Hkv, HEAD_DIM,
                 int(q_global_start), FLAG_DETERMINISTIC if deterministic else 0, 0)
    lib = library()
    mem = _workspace(lib.qsa_doc_plan_bytes(ctypes.byref(dd)), qd.device, plan_mem)
    struct = PlanStruct()
    st = lib.qsa_doc_plan_build(ctypes.byref(dd), qd.data_ptr(), kd.data_ptr(), mem.data_ptr(),
                                mem.numel() * mem.element_size(), ctypes.byref(struct),
                                _stream())
    _raise(st)
    return Plan(struct, mem)


def doc_forward(q, k, v, q_doc_ids, kv_doc_ids, scale: Optional[float] = None, *,
                q_global_start: int = 0, out=None, out_fp32=None, lse=None, workspace=None,
                deterministic: bool = False):
    """Causal attention within documents (``qsa_doc_forward``); returns
    ``(out, out_fp32, lse [B, Hq, Sq])``."""
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    if v.shape != k.shape:
        raise ValueError("v must have k's shape")
    dd, qd, kd = _doc_args(q, k, q_doc_ids, kv_doc_ids, q_global_start, deterministic)
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    out = torch.empty_like(q) if out is None else out
    out_fp32 = torch.empty(q.shape, dtype=torch.float32, device=q.device) if out_fp32 is None \
        else out_fp32
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                      device=q.device) if lse is None else lse
    lib = library()
    ws = _workspace(lib.qsa_doc_forward_workspace_bytes(ctypes.byref(dd)), q.device, workspace)
    st = lib.qsa_doc_forward(ctypes.byref(dd), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             qd.data_ptr(), kd.data_ptr(), float(scale), out.data_ptr(),
                             out_fp32.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                             ws.numel() * ws.element_size(), _stream())
    _raise(st)
    return out, out_fp32, lse


def doc_backward(grad_out, q, k, v, out_fp32, lse, q_doc_ids, kv_doc_ids,
                 scale: Optional[float] = None, *, q_global_start: int = 0, dq=None, dk=None,
                 dv=None, workspace=None, deterministic: bool = False):
    """Backward of causal attention within documents (``qsa_doc_backward``)."""
    grad_out = _check(grad_out, torch.bfloat16, "grad_out")
    q = _check(q, torch.bfloat16, "q")
    k = _check(k, torch.bfloat16, "k")
    v = _check(v, torch.bfloat16, "v")
    out_fp32 = _check(out_fp32, torch.float32, "out_fp32")
    lse = _check(lse, torch.float32, "lse")
    dd, qd, kd = _doc_args(q, k, q_doc_ids, kv_doc_ids, q_global_start, deterministic)
    if grad_out.shape != q.shape or out_fp32.shape != q.shape:
        raise ValueError("grad_out and out_fp32 must have q's shape")
    if lse.shape != (q.shape[0], q.shape[2], q.shape[1]):
        raise ValueError("lse must be [B, Hq, Sq]")
    if scale is None:
        scale = 1.0 / (q.shape[-1] ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = library()
    ws = _workspace(lib.qsa_doc_backward_workspace_bytes(ctypes.byref(dd)), q.device, workspace)
    st = lib.qsa_doc_backward(ctypes.byref(dd), grad_out.data_ptr(), q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), out_fp32.data_ptr(), lse.data_ptr(), qd.data_ptr(),
                              kd.data_ptr(), float(scale), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                              _stream())
    _raise(st)
    return dq, dk, dv


def select_dims(q_idx: torch.Tensor, kbar: torch.Tensor, top_k: int, q_offset: int = 0,
                flags: int = 0) -> SelectDims:
    """``qsa_select_dims`` for q_idx [B, Sq, H, D] and kbar [B, NB, D]."""
    if q_idx.dim() != 4 or kbar.dim() != 3:
        raise ValueError("q_idx must be [B, Sq, H, D] and kbar [B, NB, D]")
    B, Sq, H, D = q_idx.shape
    if kbar.shape[0] != B or kbar.shape[2] != D:
        raise ValueError("kbar must be [B, NB, D] with q_idx's B and D")
    return SelectDims(B, Sq, kbar.shape[1], q_offset, H, D, top_k, flags)


def select(q_idx, kbar, top_k: int, scale: Optional[float] = None, *, q_offset: int = 0,
           doc_start=None, blk_base=None, blocks: bool = True, routes: bool = True,
           scores: bool = False, workspace=None):
    """Block selector (``qsa_select``): scores every visible compressed block,
    keeps each query's top_k and expands them to route rows. Returns
    ``(blocks [B, Sq, top_k] | None, routes [B, Sq, 4 top_k + 4] | None,
    scores [B, Sq, NB] | None)``, each only when asked for."""
    q_idx = _check(q_idx, torch.bfloat16, "q_idx")
    kbar = _check(kbar, torch.bfloat16, "kbar")
    sd = select_dims(q_idx, kbar, top_k, q_offset)
    B, Sq = q_idx.shape[:2]
    meta = []
    for name, m in (("doc_start", doc_start), ("blk_base", blk_base)):
        if m is not None:
            m = _check(m, torch.int32, name)
            if m.shape != (B, Sq):
                raise ValueError(f"{name} must be [B, Sq] int32")
        meta.append(m)
    if scale is None:
        scale = 1.0 / (q_idx.shape[-1] ** 0.5)
    dev = q_idx.device
    bo = torch.empty((B, Sq, top_k), dtype=torch.int32, device=dev) if blocks else None
    ro = torch.empty((B, Sq, 4 * top_k + 4), dtype=torch.int32, device=dev) if routes else None
    so = torch.empty((B, Sq, kbar.shape[1]), dtype=torch.float32, device=dev) if scores else None
    lib = library()
    if so is None:
        ws = _workspace(lib.qsa_select_workspace_bytes(ctypes.byref(sd)), dev, workspace)
        ws_ptr, ws_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    st = lib.qsa_select(ctypes.byref(sd), q_idx.data_ptr(), kbar.data_ptr(), _ptr(meta[0]),
                        _ptr(meta[1]), float(scale), _ptr(bo), _ptr(ro), _ptr(so), ws_ptr,
                        ws_bytes, _stream())
    _raise(st)
    return bo, ro, so
