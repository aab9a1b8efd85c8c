"""FP64 CPU oracle for route-set grouped-query attention (QSA).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product library
never imports, links or runs anything in this package, and this package never
imports the product.

The attention arithmetic lives in ``qsa_oracle.c`` (plain loops, double
precision, OpenMP over rows); this module compiles it with gcc on first use,
widens the bf16 inputs exactly to float64 and marshals arrays through ctypes.
The block selector (``select_*``) is plain numpy in float64 in this module.
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
                ("dout", ctypes.c_void_p), ("o_saved", ctypes.c_void_p),
                ("lse_saved", ctypes.c_void_p)]


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
        lib.orc_block_membership.restype = None
        lib.orc_block_membership.argtypes = [P, I, I, P, P, P, P, I, I, P, P]
        lib.orc_doc_membership.restype = None
        lib.orc_doc_membership.argtypes = [P, P, I, I, I, I, I, P, P]
        lib.orc_tiles.restype = None
        lib.orc_tiles.argtypes = [P, I, I, I, I, I, I] + [P] * 9
        for name in ("orc_forward", "orc_backward_dq"):
            getattr(lib, name).restype = None
        lib.orc_forward.argtypes = [ctypes.POINTER(_Problem), I, P, P, P]
        lib.orc_backward_dq.argtypes = [ctypes.POINTER(_Problem), I, P, P]
        lib.orc_backward_dkdv.restype = None
        lib.orc_backward_dkdv.argtypes = [ctypes.POINTER(_Problem), I, P, P, P]
        lib.orc_backward_rows.restype = None
        lib.orc_backward_rows.argtypes = [ctypes.POINTER(_Problem), I, P, P, P, P, P, P]
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


def block_membership(sel_blocks: np.ndarray, lo: np.ndarray, hi: np.ndarray,
                     blk_base: np.ndarray, tok_base: np.ndarray,
                     block_size: int = 4) -> tuple[np.ndarray, np.ndarray]:
    """Byte membership ``[1, T, stride]`` and ``has_routes`` ``[1, T]`` of a block-bitmap
    selection over T packed tokens (the lookup of the cuDNN Frontend QSA page,
    "Selection and components"); ``sel_blocks`` is uint8 ``[T, NB]``, the rest int32."""
    sel = np.ascontiguousarray(sel_blocks, dtype=np.uint8)
    T, NB = sel.shape
    meta = [np.ascontiguousarray(a, dtype=np.int32) for a in (lo, hi, blk_base, tok_base)]
    assert all(a.shape == (T,) for a in meta)
    stride = row_stride(T)
    memb = np.empty((1, T, stride), dtype=np.uint8)
    has = np.empty((1, T), dtype=np.uint8)
    _load().orc_block_membership(_ptr(sel), T, NB, *[_ptr(a) for a in meta], block_size, stride,
                                 _ptr(memb), _ptr(has))
    return memb, has


def doc_membership(q_doc: np.ndarray, kv_doc: np.ndarray,
                   q_global_start: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Byte membership ``[B, Sq, stride]`` and ``has_routes`` ``[B, Sq]`` of causal
    attention within documents: query i (global position q_global_start + i) sees key
    j iff its document id is nonzero, equals key j's, and j <= its position ("fa4"
    page, ``document_causal_fa4_attention``)."""
    qd = np.ascontiguousarray(q_doc, dtype=np.int32)
    kd = np.ascontiguousarray(kv_doc, dtype=np.int32)
    B, Sq = qd.shape
    Skv = kd.shape[1]
    assert kd.shape[0] == B
    stride = row_stride(Skv)
    memb = np.empty((B, Sq, stride), dtype=np.uint8)
    has = np.empty((B, Sq), dtype=np.uint8)
    _load().orc_doc_membership(_ptr(qd), _ptr(kd), B, Sq, Skv, q_global_start, stride,
                               _ptr(memb), _ptr(has))
    return memb, has


def routes_from_membership(memb: np.ndarray, Skv: int) -> np.ndarray:
    """Route rows listing each row's members in ascending order, -1 padded: the same
    sets as ``memb``, for building a :class:`Problem`."""
    B, Sq, _ = memb.shape
    m = memb[:, :, :Skv].reshape(B * Sq, Skv) != 0
    cnt = m.sum(axis=1)
    W = max(int(cnt.max()) if cnt.size else 0, 1)
    routes = np.full((B * Sq, W), -1, dtype=np.int32)
    rows, cols = np.nonzero(m)
    pos = np.arange(rows.size) - np.repeat(np.cumsum(cnt) - cnt, cnt)
    routes[rows, pos] = cols
    return routes.reshape(B, Sq, W)


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
        self.o_saved = self.lse_saved = None
        self._c = _Problem(B, Sq, Skv, Hq, Hkv, D, self.W, self.i64, 0, self.scale,
                           _ptr(self.routes), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                           _ptr(self.dout) if self.dout is not None else 0, 0, 0)

    def use_saved(self, out, lse) -> "Problem":
        """Make the backward take this O ``[B, Sq, Hq, D]`` and LSE ``[B, Hq, Sq]`` (for
        instance a GPU forward's out_fp32 and lse) instead of the oracle's own forward;
        ``None`` restores the oracle's own."""
        if out is None:
            self.o_saved = self.lse_saved = None
            self._c.o_saved = self._c.lse_saved = 0
            return self
        out = np.ascontiguousarray(out, dtype=np.float64)
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        if out.shape != (self.B, self.Sq, self.Hq, self.D) or lse.shape != (self.B, self.Hq,
                                                                              self.Sq):
            raise ValueError("saved out must be [B, Sq, Hq, D] and lse [B, Hq, Sq]")
        self.o_saved, self.lse_saved = out, lse
        self._c.o_saved, self._c.lse_saved = _ptr(out), _ptr(lse)
        return self

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
                                  _ptr(dk), _ptr(dv), None, None)
        return dq, dk, dv

    def all_outputs(self):
        """Forward and full backward in one pass over every row:
        out [B, Sq, Hq, D], lse [B, Hq, Sq], dq [B, Sq, Hq, D], dk, dv [B, Skv, Hkv, D]."""
        if self.dout is None:
            raise ValueError("grad_out missing")
        rows = self._rows(None)
        n = rows.shape[0]
        out = np.empty((n, self.Hq, self.D), np.float64)
        lse = np.empty((n, self.Hq), np.float64)
        dq = np.empty((n, self.Hq, self.D), np.float64)
        dk = np.empty((self.B, self.Skv, self.Hkv, self.D), np.float64)
        dv = np.empty_like(dk)
        _load().orc_backward_rows(ctypes.byref(self._c), n, _ptr(rows), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(out), _ptr(lse))
        shp = (self.B, self.Sq, self.Hq, self.D)
        return (out.reshape(shp), lse.reshape(self.B, self.Sq, self.Hq).transpose(0, 2, 1).copy(),
                dq.reshape(shp), dk, dv)

    def backward_full(self):
        """dq [B, Sq, Hq, D], dk, dv [B, Skv, Hkv, D]."""
        dq, dk, dv = self.backward_rows()
        return dq.reshape(self.B, self.Sq, self.Hq, self.D), dk, dv



# ---- block selector (cuDNN Frontend QSA page, "Finding QSA attention and its
# indexer"; route format: NeMo AutoModel QSA page, `cudnn_sparse_gqa_attention`
# and the routes parameter of the packed-coordinate translation) ----

def _select_meta(B: int, Sq: int, doc_start, blk_base):
    s = np.zeros((B, Sq), np.int64) if doc_start is None else np.asarray(doc_start, np.int64)
    base = np.zeros((B, Sq), np.int64) if blk_base is None else np.asarray(blk_base, np.int64)
    return s, base


def select_visible(B: int, Sq: int, NB: int, q_offset: int = 0, doc_start=None,
                   blk_base=None) -> tuple[np.ndarray, np.ndarray]:
    """Which compressed blocks each query may score. Query t of batch row b sits at
    position p = q_offset + t; its document starts at s = doc_start[b, t] (0 without
    metadata) and block j of the document (tokens s + 4j .. s + 4j + 3) is row
    blk_base[b, t] + j of kbar[b] (j without metadata). A block is visible when it is
    complete before the query's own block, j < (p - s) // 4, and its row exists,
    0 <= row < NB. A query with s < 0 or s > p is padding and sees nothing.
    Returns (visible [B, Sq, NB] bool over kbar rows, c [B, Sq] = (p - s) // 4 or -1
    for padding)."""
    s, base = _select_meta(B, Sq, doc_start, blk_base)
    p = q_offset + np.arange(Sq, dtype=np.int64)[None, :]
    pad = (s < 0) | (s > p)
    c = np.where(pad, -1, (p - s) // 4)
    r = np.arange(NB, dtype=np.int64)[None, None, :]
    j = r - base[:, :, None]
    vis = (j >= 0) & (j < c[:, :, None])
    return vis, c


def select_scores(q_idx: np.ndarray, kbar: np.ndarray, scale: float, q_offset: int = 0,
                  doc_start=None, blk_base=None) -> np.ndarray:
    """Block scores in FP64: scale * sum over heads h of relu(q_idx[b, t, h] . kbar[b, r])
    for every visible kbar row r (see select_visible), -inf elsewhere. q_idx [B, Sq, H, d]
    and kbar [B, NB, d], bf16 bit patterns (widened exactly) or float arrays; returns
    [B, Sq, NB] indexed by kbar row."""
    q = widen(q_idx) if q_idx.dtype == np.uint16 else np.asarray(q_idx, np.float64)
    k = widen(kbar) if kbar.dtype == np.uint16 else np.asarray(kbar, np.float64)
    B, Sq = q.shape[:2]
    NB = k.shape[1]
    vis, _ = select_visible(B, Sq, NB, q_offset, doc_start, blk_base)
    out = np.full((B, Sq, NB), -np.inf)
    for b in range(B):
        dots = np.matmul(q[b], k[b].T)                     # [Sq, H, NB]: every head's dot
        score = scale * np.maximum(dots, 0.0).sum(axis=1)   # relu per head, then the sum
        out[b] = np.where(vis[b], score, -np.inf)
    return out


def select_blocks(scores: np.ndarray, top_k: int, q_offset: int = 0, doc_start=None,
                  blk_base=None) -> np.ndarray:
    """The selector's output, local block numbers [B, Sq, top_k]: per query the top_k
    visible blocks by score (all of them when fewer are visible), listed in ascending
    order and padded with -1. Blocks of equal score rank by block number, the lower
    first (the pages leave the tie rule open)."""
    B, Sq, NB = scores.shape
    vis, _ = select_visible(B, Sq, NB, q_offset, doc_start, blk_base)
    _, base = _select_meta(B, Sq, doc_start, blk_base)
    out = np.full((B, Sq, top_k), -1, np.int32)
    for b in range(B):
        for t in range(Sq):
            rows = np.nonzero(vis[b, t])[0]
            ranked = sorted(rows.tolist(), key=lambda r: (-scores[b, t, r], r))
            chosen = np.sort(np.array(ranked[:top_k], np.int64)) - base[b, t]
            out[b, t, :len(chosen)] = chosen
    return out


def select_routes(blocks: np.ndarray, q_offset: int = 0, doc_start=None) -> np.ndarray:
    """Expansion of the selector's block numbers to route rows [B, Sq, 4 top_k + 4]: the
    chosen blocks' token IDs s + 4j .. s + 4j + 3 in the order given, -1 for unused
    slots, then the query's own incomplete block, tokens s + 4((p - s) // 4) .. p,
    padded with -1 to four slots. Padding queries get a row of -1."""
    B, Sq, top_k = blocks.shape
    s, _ = _select_meta(B, Sq, doc_start, None)
    out = np.full((B, Sq, 4 * top_k + 4), -1, np.int32)
    for b in range(B):
        for t in range(Sq):
            p, st = q_offset + t, int(s[b, t])
            if st < 0 or st > p:
                continue
            for n, j in enumerate(blocks[b, t]):
                if j >= 0:
                    out[b, t, 4 * n:4 * n + 4] = st + 4 * j + np.arange(4)
            own = np.arange(st + 4 * ((p - st) // 4), p + 1)
            out[b, t, 4 * top_k:4 * top_k + len(own)] = own
    return out
