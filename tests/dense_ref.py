"""Dense brute-force route-set attention in NumPy float64 (for pinning the oracle).

This is a second, independent formulation of the same definition: the routes
are scattered into a dense boolean mask with fancy indexing, and attention is a
dense masked softmax over all keys with whole-matrix products. Rows with no
allowed key are special-cased to output 0 and lse -inf. It is only used on tiny
inputs.
"""
from __future__ import annotations

import numpy as np


def dense_mask(routes: np.ndarray, Skv: int) -> np.ndarray:
    r = routes.astype(np.int64)
    B, Sq, W = r.shape
    m = np.zeros((B, Sq, Skv), dtype=bool)
    valid = (r >= 0) & (r < Skv)
    b, i, w = np.nonzero(valid)
    m[b, i, r[b, i, w]] = True
    return m


def _expand(k: np.ndarray, Hq: int) -> np.ndarray:
    return np.repeat(k, Hq // k.shape[2], axis=2)


def dense_forward(q, k, v, mask, scale):
    """q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D], mask [B,Sq,Skv] -> out [B,Sq,Hq,D], lse [B,Hq,Sq]."""
    Hq = q.shape[2]
    kk, vv = _expand(k, Hq), _expand(v, Hq)
    s = scale * np.einsum("bihd,bjhd->bhij", q, kk)
    m4 = np.broadcast_to(mask[:, None], s.shape)
    s = np.where(m4, s, -np.inf)
    empty = ~m4.any(-1)
    mx = np.where(empty, 0.0, s.max(-1))
    e = np.where(m4, np.exp(s - mx[..., None]), 0.0)
    l = e.sum(-1)
    lse = np.where(empty, -np.inf, mx + np.log(np.where(empty, 1.0, l)))
    p = np.where(m4, e / np.where(empty, 1.0, l)[..., None], 0.0)
    out = np.einsum("bhij,bjhd->bihd", p, vv)
    return out, lse


def dense_backward(q, k, v, dout, mask, scale, out=None, lse=None):
    """Closed-form gradients of the dense masked softmax attention. ``out`` and
    ``lse`` replace the forward's own O and LSE when given (saved state)."""
    B, Sq, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    kk, vv = _expand(k, Hq), _expand(v, Hq)
    if out is None:
        out, lse = dense_forward(q, k, v, mask, scale)
    s = scale * np.einsum("bihd,bjhd->bhij", q, kk)
    m4 = np.broadcast_to(mask[:, None], s.shape)
    p = np.where(m4, np.exp(s - np.where(np.isfinite(lse), lse, 0.0)[..., None]), 0.0)
    delta = np.einsum("bihd,bihd->bhi", dout, out)
    dp = np.einsum("bihd,bjhd->bhij", dout, vv)
    ds = p * (dp - delta[..., None])
    dq = scale * np.einsum("bhij,bjhd->bihd", ds, kk)
    dk_h = scale * np.einsum("bhij,bihd->bjhd", ds, q)
    dv_h = np.einsum("bhij,bihd->bjhd", p, dout)
    dk = dk_h.reshape(B, -1, Hkv, G, D).sum(3)
    dv = dv_h.reshape(B, -1, Hkv, G, D).sum(3)
    return dq, dk, dv
