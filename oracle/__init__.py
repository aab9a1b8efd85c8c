"""FP64 CPU oracle for route-set grouped-query attention (QSA).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product library
never imports, links or runs anything in this package, and this package never
imports the product.

The arithmetic lives in ``qsa_oracle.c`` (plain loops, double precision,
OpenMP over rows); this module compiles it with gcc on first use, widens the
bf16 inputs exactly to float64 and marshals arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "libqsa_oracle.so")
_lib = None

TILE = 128


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libqsa_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64),
                ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64), ("D", ctypes.c_int64),
                ("W", ctypes.c_int64), ("route_is_i64", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("scale", ctypes.c_double), ("routes", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("dout", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.orc_route_set.restype = I
        lib.orc_route_set.argtypes = [P, ctypes.c_int32, I, I, I, P]
        lib.orc_membership.restype = None
        lib.orc_membership.argtypes = [P, ctypes.c_int32, I, I, I, I, I, P, P]
        lib.orc_tiles.restype = None
        lib.orc_tiles.argtypes = [P, I, I, I, I, I, I] + [P] * 9
        for name in ("orc_forward", "orc_backward_dq"):
            getattr(lib, name).restype = None
        lib.orc_forward.argtypes = [ctypes.POINTER(_Problem), I, P, P, P]
        lib.orc_backward_dq.argtypes = [ctypes.POINTER(_Problem), I, P, P]
        lib.orc_backward_dkdv.restype = None
        lib.orc_backward_dkdv.argtypes = [ctypes.POINTER(_Problem), I, P, P, P]
        lib.orc_backward_rows.restype = None
        lib.orc_backward_rows.argtypes = [ctypes.POINTER(_Problem), I, P, P, P, P]
        lib.orc_num_threads.restype = ctypes.c_int32
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def widen(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float arrays -> contiguous float64."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _routes(routes: np.ndarray) -> tuple[np.ndarray, int]:
    if routes.dtype == np.int64:
        return np.ascontiguousarray(routes), 1
    if routes.dtype == np.int32:
        return np.ascontiguousarray(routes), 0
    raise TypeError("routes must be int32 or int64")


def row_stride(Skv: int) -> int:
    """Membership row stride: Skv rounded up to a multiple of 128 bytes."""
    return (Skv + TILE - 1) // TILE * TILE


def route_set(routes: np.ndarray, Skv: int, row: int) -> np.ndarray:
    r, i64 = _routes(routes)
    W = r.shape[-1]
    keys = np.empty(max(W, 1), dtype=np.int64)
    n = _load().orc_route_set(_ptr(r), i64, W, Skv, row, _ptr(keys))
    return keys[:n].copy()


def membership(routes: np.ndarray, Skv: int) -> tuple[np.ndarray, np.ndarray]:
    """Byte membership ``[B, Sq, stride]`` and ``has_routes`` ``[B, Sq]``."""
    r, i64 = _routes(routes)
    B, Sq, W = r.shape
    stride = row_stride(Skv)
    memb = np.empty((B, Sq, stride), dtype=np.uint8)
    has = np.empty((B, Sq), dtype=np.uint8)
    _load().orc_membership(_ptr(r), i64, B, Sq, W, Skv, stride, _ptr(memb), _ptr(has))
    return memb, has


def tiles(memb: np.ndarray, Skv: int, tq: int = TILE, tk: int = TILE) -> dict:
    """Tile kinds and forward/reverse partial/full lists from a membership table."""
    memb = np.ascontiguousarray(memb, dtype=np.uint8)
    B, Sq, stride = memb.shape
    nqt, nkt = -(-Sq // tq), -(-Skv // tk)
    out = {
        "kinds": np.empty((B, nqt, nkt), np.int32),
        "fwd_p_cnt": np.empty((B, nqt), np.int32), "fwd_p_idx": np.empty((B, nqt, nkt), np.int32),
        "fwd_f_cnt": np.empty((B, nqt), np.int32), "fwd_f_idx": np.empty((B, nqt, nkt), np.int32),
        "rev_p_cnt": np.empty((B, nkt), np.int32), "rev_p_idx": np.empty((B, nkt, nqt), np.int32),
        "rev_f_cnt": np.empty((B, nkt), np.int32), "rev_f_idx": np.empty((B, nkt, nqt), np.int32),
    }
    order = ["kinds", "fwd_p_cnt", "fwd_p_idx", "fwd_f_cnt", "fwd_f_idx", "rev_p_cnt",
             "rev_p_idx", "rev_f_cnt", "rev_f_idx"]
    _load().orc_tiles(_ptr(memb), B, Sq, Skv, stride, tq, tk, *[_ptr(out[n]) for n in order])
    return out


class Problem:
    """Holds widened inputs for repeated oracle calls."""

    def __init__(self, q, k, v, routes, scale: float, grad_out=None):
        self.q = widen(q)
        self.k = widen(k)
        self.v = widen(v)
        self.dout = widen(grad_out) if grad_out is not None else None
        self.routes, self.i64 = _routes(routes)
        B, Sq, Hq, D = self.q.shape
        Bk, Skv, Hkv, Dk = self.k.shape
        if B != Bk or D != Dk or self.v.shape != self.k.shape or Hq % Hkv:
            raise ValueError("inconsistent shapes")
        if self.routes.shape[:2] != (B, Sq):
            raise ValueError("routes must be [B, Sq, W]")
        self.B, self.Sq, self.Skv, self.Hq, self.Hkv, self.D = B, Sq, Skv, Hq, Hkv, D
        self.W = self.routes.shape[2]
        self.scale = float(scale)
        self._c = _Problem(B, Sq, Skv, Hq, Hkv, D, self.W, self.i64, 0, self.scale,
                           _ptr(self.routes), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                           _ptr(self.dout) if self.dout is not None else 0)

    def _rows(self, rows: Optional[np.ndarray]) -> np.ndarray:
        if rows is None:
            rows = np.arange(self.B * self.Sq, dtype=np.int64)
        return np.ascontiguousarray(rows, dtype=np.int64)

    def forward(self, rows: Optional[np.ndarray] = None):
        """out [n, Hq, D] and lse [n, Hq] (float64) for flat rows b*Sq+i (all rows by default)."""
        rows = self._rows(rows)
        out = np.empty((rows.shape[0], self.Hq, self.D), np.float64)
        lse = np.empty((rows.shape[0], self.Hq), np.float64)
        _load().orc_forward(ctypes.byref(self._c), rows.shape[0], _ptr(rows), _ptr(out), _ptr(lse))
        return out, lse

    def forward_full(self):
        """out [B, Sq, Hq, D] and lse [B, Hq, Sq]."""
        out, lse = self.forward()
        return (out.reshape(self.B, self.Sq, self.Hq, self.D),
                lse.reshape(self.B, self.Sq, self.Hq).transpose(0, 2, 1).copy())

    def backward_dq(self, rows: Optional[np.ndarray] = None) -> np.ndarray:
        if self.dout is None:
            raise ValueError("grad_out missing")
        rows = self._rows(rows)
        dq = np.empty((rows.shape[0], self.Hq, self.D), np.float64)
        _load().orc_backward_dq(ctypes.byref(self._c), rows.shape[0], _ptr(rows), _ptr(dq))
        return dq

    def backward_dkdv(self, keys: np.ndarray):
        """dk, dv [n, Hkv, D] for flat keys b*Skv+j."""
        if self.dout is None:
            raise ValueError("grad_out missing")
        keys = np.ascontiguousarray(keys, dtype=np.int64)
        dk = np.empty((keys.shape[0], self.Hkv, self.D), np.float64)
        dv = np.empty_like(dk)
        _load().orc_backward_dkdv(ctypes.byref(self._c), keys.shape[0], _ptr(keys), _ptr(dk),
                                  _ptr(dv))
        return dk, dv

    def backward_rows(self, rows: Optional[np.ndarray] = None):
        """dq of the rows [n, Hq, D] and their contributions to dk, dv [B, Skv, Hkv, D]."""
        if self.dout is None:
            raise ValueError("grad_out missing")
        rows = self._rows(rows)
        dq = np.empty((rows.shape[0], self.Hq, self.D), np.float64)
        dk = np.empty((self.B, self.Skv, self.Hkv, self.D), np.float64)
        dv = np.empty_like(dk)
        _load().orc_backward_rows(ctypes.byref(self._c), rows.shape[0], _ptr(rows), _ptr(dq),
                                  _ptr(dk), _ptr(dv))
        return dq, dk, dv

    def backward_full(self):
        """dq [B, Sq, Hq, D], dk, dv [B, Skv, Hkv, D]."""
        dq, dk, dv = self.backward_rows()
        return dq.reshape(self.B, self.Sq, self.Hq, self.D), dk, dv
