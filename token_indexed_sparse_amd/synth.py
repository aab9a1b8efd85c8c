"""Seeded synthetic inputs for route-set grouped-query attention.

This module only draws random numbers and lays out route slots. It holds none
of the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method.

Route rows follow the shape of the routes a ratio-four block indexer emits
("cuDNN Frontend indexed QSA training" page, ``_pack_indices`` and
``cudnn_sparse_gqa_attention``): groups of four slots that each hold one
distinct complete four-token block, plus the query's own incomplete causal
block, padded with -1. Block numbering restarts at every document origin.

Slot layout of one row (width ``W = 4 * n_max + 4``)::

    [complete blocks in ascending order, 4 IDs each]
    [-1] * 4 * (n_max - n_chosen)
    [own partial block IDs p0 .. p, -1-padded to 4]

Draw order for every workload: structure (document cuts or valid lengths),
then routes row by row in ascending (batch, position), then q, k, v, grad_out.
Floating tensors are float32 N(0, 1) rounded to bf16 with round-to-nearest-even
and are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and route recipe of one synthetic workload."""

    name: str
    B: int
    Sq: int
    Skv: int
    Hq: int
    Hkv: int
    D: int
    n_max: int           # complete blocks per row at most
    kind: str            # route recipe, see ``make_routes``
    seed: int
    q_offset: int = 0    # global position of local query 0 (context-parallel shard)
    n_docs: int = 1      # packed documents per row ("docs" recipe)
    len_lo: int = 0      # valid-length range ("padded" recipe)
    len_hi: int = 0
    recent_blocks: int = 0  # always-selected most recent blocks ("recent_earlier" recipe)

    @property
    def W(self) -> int:
        return 4 * self.n_max + 4

    @property
    def scale(self) -> float:
        return 1.0 / 16.0


# The five synthetic workloads. Seed = index.
WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_s256_12q1kv", 1, 256, 256, 12, 1, 256, 8, "single", 1),
    2: Workload("thd_t8192_4docs_12q1kv", 1, 8192, 8192, 12, 1, 256, 64, "docs", 2, n_docs=4),
    3: Workload("padded_b4_s4096_24q2kv", 4, 4096, 4096, 24, 2, 256, 64, "padded", 3,
                len_lo=1024, len_hi=4096),
    4: Workload("long_t32768_12q1kv", 1, 32768, 32768, 12, 1, 256, 512, "recent_earlier", 4,
                recent_blocks=256),
    5: Workload("cp_shard_q4096_kv32768_12q1kv", 1, 4096, 32768, 12, 1, 256, 256, "single", 5,
                q_offset=28672),
}


def _row(out: np.ndarray, n_max: int, doc_start: int, pos: int, chosen: np.ndarray,
         record: Optional[list] = None) -> None:
    """Write one route row for a query at ``pos`` in a document starting at ``doc_start``;
    with ``record``, also append (doc_start, chosen block numbers, own block number)."""
    out.fill(-1)
    chosen = np.sort(np.asarray(chosen, dtype=np.int64))
    n = chosen.shape[0]
    if n:
        ids = doc_start + 4 * chosen[:, None] + np.arange(4, dtype=np.int64)[None, :]
        out[: 4 * n] = ids.reshape(-1)
    c = (pos - doc_start) // 4
    own = np.arange(doc_start + 4 * c, pos + 1, dtype=np.int64)
    out[4 * n_max: 4 * n_max + own.shape[0]] = own
    if record is not None:
        record.append((doc_start, chosen, c))


def _choose(rng: np.random.Generator, population: int, k: int) -> np.ndarray:
    """``k`` distinct block numbers from ``range(population)``; no draw when k == 0."""
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    return rng.choice(population, k, replace=False)


def make_routes(wl: Workload, rng: np.random.Generator,
                record_blocks: bool = False) -> tuple[np.ndarray, dict]:
    """Draw the route tensor ``[B, Sq, W]`` (int32) for ``wl``; return it and the structure.

    With ``record_blocks``, ``info["row_blocks"][b * Sq + i]`` holds the row's
    (doc_start, chosen complete block numbers, own block number), None for a row
    without routes; the draws are the same either way."""
    B, Sq, W, n_max = wl.B, wl.Sq, wl.W, wl.n_max
    routes = np.full((B, Sq, W), -1, dtype=np.int32)
    row = np.empty(W, dtype=np.int64)
    info: dict = {}
    rec: Optional[list] = [] if record_blocks else None
    if rec is not None:
        info["row_blocks"] = rec
    if wl.kind == "single":
        for b in range(B):
            for i in range(Sq):
                p = wl.q_offset + i
                c = p // 4
                _row(row, n_max, 0, p, _choose(rng, c, min(n_max, c)), rec)
                routes[b, i] = row
    elif wl.kind == "docs":
        assert B == 1 and wl.q_offset == 0
        cuts = np.sort(rng.choice(np.arange(1, Sq), wl.n_docs - 1, replace=False))
        starts = np.concatenate([[0], cuts]).astype(np.int64)
        info["doc_starts"] = starts
        doc_of = np.searchsorted(starts, np.arange(Sq), side="right") - 1
        for i in range(Sq):
            s = int(starts[doc_of[i]])
            c = (i - s) // 4
            _row(row, n_max, s, i, _choose(rng, c, min(n_max, c)), rec)
            routes[0, i] = row
    elif wl.kind == "padded":
        lengths = np.array([rng.integers(wl.len_lo, wl.len_hi, endpoint=True) for _ in range(B)],
                           dtype=np.int64)
        info["lengths"] = lengths
        for b in range(B):
            for i in range(int(lengths[b])):
                c = i // 4
                _row(row, n_max, 0, i, _choose(rng, c, min(n_max, c)), rec)
                routes[b, i] = row
            if rec is not None:
                rec.extend([None] * (Sq - int(lengths[b])))
    elif wl.kind == "recent_earlier":
        R = wl.recent_blocks
        for b in range(B):
            for i in range(Sq):
                c = i // 4
                lo = max(0, c - R)
                recent = np.arange(lo, c, dtype=np.int64)
                earlier = _choose(rng, lo, min(n_max - R, lo))
                _row(row, n_max, 0, i, np.concatenate([earlier, recent]), rec)
                routes[b, i] = row
    else:
        raise ValueError(f"unknown route recipe {wl.kind!r}")
    return routes, info


@dataclasses.dataclass
class Inputs:
    wl: Workload
    routes: np.ndarray      # int32 [B, Sq, W]
    q: np.ndarray           # uint16 (bf16 bits) [B, Sq, Hq, D]
    k: np.ndarray           # uint16 [B, Skv, Hkv, D]
    v: np.ndarray           # uint16 [B, Skv, Hkv, D]
    grad_out: np.ndarray    # uint16 [B, Sq, Hq, D]
    info: dict


def make_inputs(wl: Workload, with_grad: bool = True, record_blocks: bool = False) -> Inputs:
    """All inputs of workload ``wl``, drawn from ``numpy.random.default_rng(wl.seed)``."""
    rng = np.random.default_rng(wl.seed)
    routes, info = make_routes(wl, rng, record_blocks)
    q = bf16_bits(rng.standard_normal((wl.B, wl.Sq, wl.Hq, wl.D), dtype=np.float32))
    k = bf16_bits(rng.standard_normal((wl.B, wl.Skv, wl.Hkv, wl.D), dtype=np.float32))
    v = bf16_bits(rng.standard_normal((wl.B, wl.Skv, wl.Hkv, wl.D), dtype=np.float32))
    go = (bf16_bits(rng.standard_normal((wl.B, wl.Sq, wl.Hq, wl.D), dtype=np.float32))
          if with_grad else None)
    return Inputs(wl, routes, q, k, v, go, info)


def random_case(seed: int, B: int, Sq: int, Skv: int, Hq: int, Hkv: int, W: int,
                D: int = 256, p_pad: float = 0.2, p_dup: float = 0.1, p_bad: float = 0.05,
                empty_rows: int = 2, causal: bool = False, route_dtype=np.int32) -> Inputs:
    """Arbitrary token sets with padding, duplicates and out-of-range IDs.

    Each slot independently holds a uniform key in ``[0, Skv)`` (``[0, i]`` when
    ``causal``), a copy of an earlier slot of its row (``p_dup``), ``-1``
    (``p_pad``) or an out-of-range value (``p_bad``: ``Skv``, ``Skv + 7``,
    ``-5``, the most negative value of the dtype, and for int64 also values of
    the form ``2**32 + r``). ``empty_rows`` rows per batch are all ``-1``.
    """
    rng = np.random.default_rng(seed)
    routes = rng.integers(0, Skv, size=(B, Sq, W), dtype=np.int64)
    if causal:
        lim = np.minimum(np.arange(Sq), Skv - 1)[None, :, None] + 1
        routes = np.floor(rng.random((B, Sq, W)) * lim).astype(np.int64)
    u = rng.random((B, Sq, W))
    dup_src = rng.integers(0, W, size=(B, Sq, W))
    for w in range(1, W):
        m = (u[:, :, w] < p_dup)
        src = np.minimum(dup_src[:, :, w], w - 1)
        routes[:, :, w] = np.where(m, np.take_along_axis(routes, src[:, :, None], 2)[:, :, 0],
                                   routes[:, :, w])
    bad_vals = [Skv, Skv + 7, -5, np.iinfo(route_dtype).min]
    if route_dtype == np.int64:
        bad_vals += [2**32 + 5, 2**40 + 1, np.iinfo(np.int64).max]
    bad = rng.choice(np.array(bad_vals, dtype=np.int64), size=(B, Sq, W))
    routes = np.where((u >= p_dup) & (u < p_dup + p_bad), bad, routes)
    routes = np.where((u >= p_dup + p_bad) & (u < p_dup + p_bad + p_pad), -1, routes)
    for b in range(B):
        rows = rng.choice(Sq, min(empty_rows, Sq), replace=False)
        routes[b, rows, :] = -1
    routes = routes.astype(route_dtype)
    q = bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    k = bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    v = bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    go = bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    wl = Workload(f"random_{seed}", B, Sq, Skv, Hq, Hkv, D, (W - 4) // 4 if W >= 4 else 0,
                  "random", seed)
    return Inputs(wl, routes, q, k, v, go, {"W": W})


def tiled_case(seed: int, B: int, Sq: int, Skv: int, Hq: int, Hkv: int, p_full: float = 0.5,
               extra: int = 16, D: int = 256, bare_rows: bool = False, loud_keys: float = 0.0,
               all_keys: bool = False, causal: bool = False, loud_last: bool = False) -> Inputs:
    """Routes that select whole 128 x 128 tiles, so that full tiles occur.

    Each (batch, query tile, key tile) is chosen with probability ``p_full``
    (``all_keys``: every one; ``causal``: key tiles at or below the query
    tile, the diagonal one only up to the row's own position); every row then
    selects all keys of its chosen tiles plus ``extra`` uniform keys. With
    ``bare_rows`` the odd query tiles of batch 0 get no extra keys. Route slots
    are shuffled; spare slots hold -1, a duplicate and an out-of-range value.
    ``loud_keys`` > 0 multiplies the K rows of the first chosen key tile of
    batch 0 by that factor (large scores there); with ``loud_last`` the last
    chosen key tile instead, so that the large scores come after smaller ones
    in every row's key order.
    """
    rng = np.random.default_rng(seed)
    nQT, nKT = -(-Sq // 128), -(-Skv // 128)
    chosen = rng.random((B, nQT, nKT)) < p_full
    if all_keys:
        chosen[:] = True
    if causal:
        chosen = np.broadcast_to(np.arange(nKT)[None, :] <= np.arange(nQT)[:, None],
                                 (B, nQT, nKT)).copy()
    per_row = []
    for b in range(B):
        for i in range(Sq):
            r = i // 128
            parts = []
            for t in np.nonzero(chosen[b, r])[0]:
                hi = min(128 * t + 128, Skv)
                if causal and t == r:
                    hi = min(hi, i + 1)
                parts.append(np.arange(128 * t, hi))
            n_extra = 0 if (bare_rows and b == 0 and r % 2 == 1) else extra
            parts.append(rng.integers(0, Skv, n_extra))
            per_row.append(np.concatenate(parts).astype(np.int64))
    W = max(len(k) for k in per_row) + 3
    routes = np.full((B, Sq, W), -1, np.int64)
    for idx, keys in enumerate(per_row):
        b, i = divmod(idx, Sq)
        vals = np.full(W, -1, np.int64)
        vals[:len(keys)] = keys
        vals[len(keys)] = keys[0] if len(keys) else -1
        vals[len(keys) + 1] = Skv + 3
        routes[b, i, rng.permutation(W)] = vals
    routes = routes.astype(np.int32)
    q = bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    kf = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    if loud_keys > 0:
        t0 = np.nonzero(chosen[0].any(axis=0))[0]
        if len(t0):
            tl = t0[-1] if loud_last else t0[0]
            kf[0, 128 * tl:128 * tl + 128] *= loud_keys
    k = bf16_bits(kf)
    v = bf16_bits(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32))
    go = bf16_bits(rng.standard_normal((B, Sq, Hq, D), dtype=np.float32))
    wl = Workload(f"tiled_{seed}", B, Sq, Skv, Hq, Hkv, D, 0, "tiled", seed)
    return Inputs(wl, routes, q, k, v, go, {"W": W})


@dataclasses.dataclass
class BlockInputs:
    """A workload in the packed block-bitmap form: T packed tokens, NB blocks."""
    T: int
    NB: int
    sel_blocks: np.ndarray   # uint8 [T, NB]
    lo: np.ndarray           # int32 [T], inclusive allowed key-token bounds
    hi: np.ndarray
    blk_base: np.ndarray     # int32 [T], first block of the query's sequence
    tok_base: np.ndarray     # int32 [T], first token of the query's sequence
    block_first: np.ndarray  # int32 [NB], inclusive token span of each block
    block_last: np.ndarray
    q: np.ndarray            # uint16 [1, T, Hq, D]
    k: np.ndarray            # uint16 [1, T, Hkv, D]
    v: np.ndarray
    grad_out: np.ndarray
    routes: np.ndarray       # int32 [1, T, W]: the same selection as packed route rows


def block_inputs(inp: Inputs) -> BlockInputs:
    """Re-express a workload drawn with ``record_blocks`` as packed sequences with a
    block-selection bitmap (the Miles packed-training layout of the cuDNN Frontend
    QSA page, "Tensors"): batch b's positions become tokens b * Sq + i; every
    document of a batch row is a sequence with its own block numbering (four
    tokens per block from the document's first token, the last block possibly
    shorter); a row selects the blocks its routes were drawn from, including its
    own incomplete block; lo is its sequence's first token and hi its own token.
    Rows without routes get lo = 0, hi = -1 and no selected block. The bitmap is
    built from the drawn block numbers, never from the route values."""
    wl = inp.wl
    rec = inp.info.get("row_blocks")
    if rec is None:
        raise ValueError("draw the workload with record_blocks=True")
    if wl.Sq != wl.Skv or wl.q_offset != 0:
        raise ValueError("the packed form needs as many keys as queries and no query offset")
    B, Sq = wl.B, wl.Sq
    T = B * Sq
    starts = [int(x) for x in inp.info.get("doc_starts", [0])]
    # sequences: (batch, start, end) in token order, with their first block
    seqs = []
    nb = 0
    for b in range(B):
        bounds = starts + [Sq]
        for s0, s1 in zip(bounds[:-1], bounds[1:]):
            seqs.append((b, s0, s1, nb))
            nb += -(-(s1 - s0) // 4)
    NB = nb
    block_first = np.empty(NB, np.int32)
    block_last = np.empty(NB, np.int32)
    base_of = {}
    for b, s0, s1, bb in seqs:
        n = -(-(s1 - s0) // 4)
        first = b * Sq + s0 + 4 * np.arange(n)
        block_first[bb:bb + n] = first
        block_last[bb:bb + n] = np.minimum(first + 3, b * Sq + s1 - 1)
        base_of[(b, s0)] = bb
    sel = np.zeros((T, NB), np.uint8)
    lo = np.zeros(T, np.int32)
    hi = np.full(T, -1, np.int32)
    blk_base = np.zeros(T, np.int32)
    tok_base = np.zeros(T, np.int32)
    for t in range(T):
        b, i = divmod(t, Sq)
        s0 = max(x for x in starts if x <= i)
        bb = base_of[(b, s0)]
        blk_base[t] = bb
        tok_base[t] = b * Sq + s0
        r = rec[t]
        if r is None:
            continue
        doc_start, chosen, own = r
        assert doc_start == s0
        sel[t, bb + chosen] = 1
        sel[t, bb + own] = 1
        lo[t] = b * Sq + s0
        hi[t] = t
    W = inp.routes.shape[2]
    off = (np.arange(B, dtype=np.int64) * Sq)[:, None, None]
    r = inp.routes.astype(np.int64)
    packed = np.where((r >= 0) & (r < wl.Skv), r + off, -1).reshape(1, T, W).astype(np.int32)
    shape_q = (1, T) + inp.q.shape[2:]
    shape_k = (1, T) + inp.k.shape[2:]
    go = inp.grad_out.reshape(shape_q) if inp.grad_out is not None else None
    return BlockInputs(T, NB, sel, lo, hi, blk_base, tok_base, block_first, block_last,
                       inp.q.reshape(shape_q), inp.k.reshape(shape_k), inp.v.reshape(shape_k),
                       go, packed)
