"""Block selector (qsa_select) on an MI355X against the oracle's selector.

* Integer-valued inputs (entries in -2..2, scale 1/2): every dot and every sum
  of the kernel is an integer below 2^24, so its FP32 scores are exact and
  must equal the oracle's bit for bit; with many equal scores the tie rule
  decides most selections, and blocks and route rows must match exactly.
  Cases: several tiles and a ragged tail, a context-parallel query shard,
  heads that are not a multiple of 16, packed documents with padding queries
  and kbar rows past the end, top_k above the visible count, and rows of
  8192 and 32768 blocks (the largest NB the call takes).
* Normal inputs: scores within an error bound derived from the FP32
  arithmetic; where the oracle's k-th and (k+1)-th scores are apart by more
  than the bound the selection must be the oracle's, elsewhere a valid top-k
  within the bound.
* The full selector shape (32768 queries, 8192 blocks, 64 heads, top_k 512):
  sampled rows against the oracle, and the format of every row.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import log, to_gpu_bf16
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu

D = 128
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _ints(rng, shape):
    return synth.bf16_bits(rng.integers(-2, 3, shape).astype(np.float32))


def _normal(rng, shape):
    return synth.bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _gpu_bf16(bits):
    return to_gpu_bf16(bits)


def _meta_gpu(m):
    return None if m is None else torch.from_numpy(np.ascontiguousarray(m, np.int32)).cuda()


def _run(q, kb, top_k, scale, q_offset=0, start=None, base=None, scores=True):
    bo, ro, so = qsa.select(_gpu_bf16(q), _gpu_bf16(kb), top_k, scale, q_offset=q_offset,
                            doc_start=_meta_gpu(start), blk_base=_meta_gpu(base), scores=scores)
    torch.cuda.synchronize()
    return bo.cpu().numpy(), ro.cpu().numpy(), None if so is None else so.cpu().numpy()


def _expand(blocks, start, q_offset):
    """Route rows of block lists [B, Sq, k] (test-side, vectorized)."""
    B, Sq, k = blocks.shape
    s = np.zeros((B, Sq), np.int64) if start is None else start.astype(np.int64)
    p = q_offset + np.arange(Sq)[None, :]
    pad = (s < 0) | (s > p)
    ids = s[:, :, None, None] + 4 * blocks[:, :, :, None].astype(np.int64) + np.arange(4)
    body = np.where(blocks[:, :, :, None] >= 0, ids, -1).reshape(B, Sq, 4 * k)
    own = (s + 4 * ((p - s) // 4))[:, :, None] + np.arange(4)
    tail = np.where(own <= p[:, :, None], own, -1)
    out = np.concatenate([body, tail], axis=2)
    out[pad] = -1
    return out.astype(np.int32)


def _check_format(bo, ro, start, q_offset, n_vis, top_k):
    """Kept blocks ascending, then -1; count min(top_k, visible); routes expand them."""
    nsel = np.minimum(n_vis, top_k)
    cnt = (bo >= 0).sum(axis=2)
    assert np.array_equal(cnt, nsel), "selected count"
    idx = np.arange(top_k)[None, None, :]
    assert ((bo >= 0) == (idx < nsel[:, :, None])).all(), "-1 padding after the kept blocks"
    d = np.diff(bo, axis=2)
    assert ((d > 0) | (idx[:, :, 1:] >= nsel[:, :, None])).all(), "ascending"
    assert np.array_equal(ro, _expand(bo, start, q_offset)), "route rows"


def _docs_meta(rng, Sq, NB_slack=0, B=1, T=None, q_offset=0):
    """Packed documents over T tokens (default Sq) in each of B batch rows: for the
    queries at positions q_offset .. q_offset + Sq - 1, their document start and
    kbar row base (each row's documents' complete blocks laid end to end), ten
    padding queries per row. Returns (start, base, NB) with NB the largest row's
    block count minus NB_slack."""
    T = Sq if T is None else T
    start = np.zeros((B, Sq), np.int32)
    base = np.zeros((B, Sq), np.int32)
    nb_max = 0
    for b in range(B):
        cuts = np.sort(rng.choice(np.arange(1, T), 4, replace=False))
        starts = np.concatenate([[0], cuts])
        ends = np.concatenate([cuts, [T]])
        nblk = (ends - starts) // 4
        bases = np.concatenate([[0], np.cumsum(nblk)[:-1]])
        doc = np.searchsorted(starts, q_offset + np.arange(Sq), side="right") - 1
        start[b] = starts[doc]
        base[b] = bases[doc]
        start[b, rng.choice(Sq, 10, replace=False)] = -1     # padding queries
        nb_max = max(nb_max, int(nblk.sum()))
    return start, base, nb_max - NB_slack


INT_CASES = [
    dict(name="tiles", seed=101, B=2, Sq=300, NB=75, H=64, k=16, q_offset=0),
    dict(name="shard_h20", seed=102, B=1, Sq=200, NB=200, H=20, k=40, q_offset=600),
    dict(name="docs", seed=103, B=1, Sq=700, NB=None, H=64, k=8, q_offset=0),
    dict(name="k_above_visible", seed=104, B=1, Sq=64, NB=16, H=48, k=100, q_offset=0),
    dict(name="h1", seed=105, B=3, Sq=130, NB=40, H=1, k=3, q_offset=7),
    dict(name="nb8192", seed=106, B=1, Sq=48, NB=8192, H=16, k=512, q_offset=32768 - 48),
    dict(name="nb32768", seed=107, B=1, Sq=8, NB=32768, H=16, k=300, q_offset=4 * 32768 - 8),
    # rows of 2049..4096 and 8193..16384 blocks (16 and 64 keys per thread)
    dict(name="nb3000", seed=108, B=1, Sq=16, NB=3000, H=16, k=100, q_offset=4 * 3000 - 16),
    dict(name="nb12000", seed=109, B=1, Sq=12, NB=12000, H=16, k=1000, q_offset=4 * 12000 - 12),
    dict(name="top1", seed=110, B=2, Sq=90, NB=30, H=32, k=1, q_offset=0),
    # documents in two batch rows, and a query shard (positions 500..699) of
    # packed documents over 700 tokens
    dict(name="docs_b2", seed=116, B=2, Sq=400, NB=None, H=32, k=12, q_offset=0),
    dict(name="docs_shard", seed=117, B=1, Sq=200, NB=None, H=64, k=24, q_offset=500, T=700),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", INT_CASES, ids=lambda c: c["name"])
def test_integer_inputs_bit_exact(case):
    log(f"select case {case}")
    rng = np.random.default_rng(case["seed"])
    B, Sq, H, k, off = case["B"], case["Sq"], case["H"], case["k"], case["q_offset"]
    start = base = None
    NB = case["NB"]
    if case["name"].startswith("docs"):
        # the last rows of the largest batch row fall past kbar's end
        start, base, NB = _docs_meta(rng, Sq, NB_slack=3, B=B, T=case.get("T"), q_offset=off)
    q = _ints(rng, (B, Sq, H, D))
    kb = _ints(rng, (B, NB, D))
    bo, ro, so = _run(q, kb, k, 0.5, off, start, base)
    ref = oracle.select_scores(q, kb, 0.5, off, start, base)
    assert np.array_equal(so, ref.astype(np.float32)), "scores"
    blk = oracle.select_blocks(ref, k, off, start, base)
    assert np.array_equal(bo, blk), "blocks"
    assert np.array_equal(ro, oracle.select_routes(blk, off, start)), "routes"
    vis, _ = oracle.select_visible(B, Sq, NB, off, start, base)
    _check_format(bo, ro, start, off, vis.sum(axis=2), k)
    # equal scores really occur, and the workspace path gives the same result
    assert any(len(np.unique(r[np.isfinite(r)])) < np.isfinite(r).sum() for r in ref[0])
    bo2, ro2, _ = _run(q, kb, k, 0.5, off, start, base, scores=False)
    assert np.array_equal(bo2, bo) and np.array_equal(ro2, ro)


@pytest.mark.timeout(600)
def test_all_scores_equal_lower_blocks_win():
    """Zero compressed keys: every visible block scores 0, so each row's selection
    is decided by the tie rule alone (its first top_k blocks), with far more
    equal keys than the direct ranking takes."""
    rng = np.random.default_rng(115)
    Sq, NB, k = 24, 8192, 512
    off = 4 * NB - Sq
    q = _normal(rng, (1, Sq, 64, D))
    kb = np.zeros((1, NB, D), np.uint16)
    bo, ro, so = _run(q, kb, k, 1.0 / np.sqrt(D), off)
    c = np.minimum((off + np.arange(Sq)) // 4, NB)
    vis = np.arange(NB)[None, :] < c[:, None]
    assert (so[0][vis] == 0).all() and np.isneginf(so[0][~vis]).all()
    want = np.where(np.arange(k)[None, :] < np.minimum(c, k)[:, None], np.arange(k)[None, :], -1)
    assert np.array_equal(bo[0], want)
    assert np.array_equal(ro, _expand(bo, None, off))


def _bound(q, kb, ref, scale, H):
    """Error bound of the kernel's FP32 scores: every dot accumulates 128 exact
    products (and a zero) in FP32, the head sum adds H non-negative terms, the
    scale multiplies once; twice the first-order bound."""
    qa = np.abs(oracle.widen(q))
    ka = np.abs(oracle.widen(kb))
    absdot = np.stack([np.matmul(qa[b], ka[b].T).sum(axis=1) for b in range(q.shape[0])])
    fin = np.where(np.isfinite(ref), ref, 0.0)
    return 2.0 * U * (scale * (D + 2) * absdot + (H + 4) * fin + np.abs(fin))


def _check_selection(bo, ref, tol, k, base):
    """Rows with a clear k-th/(k+1)-th gap: the oracle's selection. Other rows: a
    valid top-k within the bound. Returns the number of rows of the second kind."""
    B, Sq, NB = ref.shape
    near = 0
    for b in range(B):
        for t in range(Sq):
            rows = np.nonzero(np.isfinite(ref[b, t]))[0]
            off = 0 if base is None else int(base[b, t])
            got = bo[b, t][bo[b, t] >= 0].astype(np.int64) + off
            if len(rows) <= k:
                assert np.array_equal(got, rows)
                continue
            sc, tl = ref[b, t, rows], tol[b, t, rows]
            order = np.argsort(-sc, kind="stable")
            want = np.sort(rows[order[:k]])
            chosen = np.isin(rows, got)
            assert chosen.sum() == k
            lo_in = (sc - tl)[order[:k]].min()
            hi_out = (sc + tl)[order[k:]].max()
            if lo_in > hi_out:
                assert np.array_equal(got, want), (b, t)
            else:
                near += 1
                assert (sc[chosen] + tl[chosen]).min() >= (sc[~chosen] - tl[~chosen]).max(), (b, t)
    return near


NORMAL_CASES = [
    dict(name="single", seed=111, B=2, Sq=256, NB=64, H=64, k=12, q_offset=0),
    dict(name="docs", seed=112, B=1, Sq=600, NB=None, H=40, k=20, q_offset=0),
    dict(name="shard", seed=113, B=1, Sq=96, NB=2048, H=64, k=256, q_offset=8192 - 96),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", NORMAL_CASES, ids=lambda c: c["name"])
def test_normal_inputs_within_bound(case):
    log(f"select case {case}")
    rng = np.random.default_rng(case["seed"])
    B, Sq, H, k, off = case["B"], case["Sq"], case["H"], case["k"], case["q_offset"]
    start = base = None
    NB = case["NB"]
    if case["name"] == "docs":
        start, base, NB = _docs_meta(rng, Sq)
    q = _normal(rng, (B, Sq, H, D))
    kb = _normal(rng, (B, NB, D))
    scale = 1.0 / np.sqrt(D)
    bo, ro, so = _run(q, kb, k, scale, off, start, base)
    ref = oracle.select_scores(q, kb, scale, off, start, base)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(so), fin) and np.isneginf(so[~fin]).all()
    tol = _bound(q, kb, ref, scale, H)
    err = np.abs(so[fin] - ref[fin])
    assert (err <= tol[fin]).all(), f"max err {err.max()} vs bound {tol[fin][err.argmax()]}"
    near = _check_selection(bo, ref, tol, k, base)
    log(f"  max |err| {err.max():.3g}, rows decided within the bound: {near}")
    vis, _ = oracle.select_visible(B, Sq, NB, off, start, base)
    _check_format(bo, ro, start, off, vis.sum(axis=2), k)


@pytest.mark.timeout(900)
def test_full_selector_shape_sampled():
    """32768 queries of one sequence, 8192 blocks, 64 indexer heads, top_k 512."""
    T, NB, H, k = 32768, 8192, 64, 512
    rng = np.random.default_rng(120)
    log("  generating inputs")
    q = _normal(rng, (1, T, H, D))
    kb = _normal(rng, (1, NB, D))
    scale = 1.0 / np.sqrt(D)
    qg, kg = _gpu_bf16(q), _gpu_bf16(kb)
    bo, ro, so = qsa.select(qg, kg, k, scale, scores=True)
    torch.cuda.synchronize()
    log("  selector ran")
    rows = np.sort(np.concatenate([[0, 3, 4, 2051, 2052, 2053, T - 1],
                                   rng.choice(T, 17, replace=False)]))
    so_s = so[0, torch.from_numpy(rows).cuda()].cpu().numpy()[None]
    bo_s = bo[0, torch.from_numpy(rows).cuda()].cpu().numpy()[None]
    ref = np.stack([oracle.select_scores(q[:, r:r + 1], kb, scale, q_offset=r)[0, 0]
                    for r in rows])[None]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(so_s), fin)
    tol = np.concatenate([_bound(q[:, r:r + 1], kb, ref[:, i:i + 1], scale, H)
                          for i, r in enumerate(rows)], axis=1)
    err = np.abs(so_s[fin] - ref[fin])
    assert (err <= tol[fin]).all()
    near = _check_selection(bo_s, ref, tol, k, None)
    log(f"  sampled rows: max |err| {err.max():.3g}, decided within the bound: {near}")
    # every row's format
    bo_all, ro_all = bo.cpu().numpy(), ro.cpu().numpy()
    n_vis = np.minimum(np.arange(T) // 4, NB)[None]
    _check_format(bo_all, ro_all, None, 0, n_vis, k)
