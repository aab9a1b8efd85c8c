"""Pins of the oracle's block selector (cuDNN Frontend QSA page, "Finding QSA
attention and its indexer": each complete compressed block scores
scale * sum_h relu(qi[t, h] . kbar[block]), the selector keeps the top k and
returns block numbers, and an expansion turns them into the route rows that the
NeMo AutoModel QSA page describes: four-token groups of complete blocks, -1
padding, then the query's incomplete causal tail).

* Hand cases: scores, selections and route rows worked out on paper from that
  statement (equal scores, an invisible own block, document metadata, a padding
  query, kbar rows past the end) and typed in.
* Closed forms: heads in +/- pairs turn the relu sum into scale * sum |q . k|;
  non-negative inputs turn it into one matrix product with the head sum of q.
* Top-k against numpy's stable argsort, and the expansion against the route
  rows of the synthetic generator (synth._row), written apart from the oracle.
"""
import numpy as np
import pytest

import oracle
from token_indexed_sparse_amd import synth

INF = np.inf

# kbar rows: (1, 0), (0, 1), (1, 1)
K3 = np.array([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]])


def _hand_q():
    q = np.zeros((1, 14, 2, 2))
    q[0, 13] = [[2, -1], [-1, 3]]   # heads: dots (2, -1, 1) and (-1, 3, 2)
    q[0, 8] = [[-1, -1], [1, -2]]   # dots (-1, -1, -2) and (1, -2, -1)
    return q


def test_hand_scores_and_selection():
    s = oracle.select_scores(_hand_q(), K3, 0.5)
    assert s.shape == (1, 14, 3)
    # positions 0..3 have no complete block before their own
    assert np.isneginf(s[0, :4]).all()
    # position 4..7: block 0 only; zero query -> score 0
    assert np.array_equal(s[0, 4], [0.0, -INF, -INF])
    # position 8: blocks 0, 1; relu sums (0 + 1, 0 + 0) * 0.5
    assert np.array_equal(s[0, 8], [0.5, 0.0, -INF])
    # position 13: blocks 0..2; relu sums (2 + 0, 0 + 3, 1 + 2) * 0.5
    assert np.array_equal(s[0, 13], [1.0, 1.5, 1.5])

    b1 = oracle.select_blocks(s, 1)
    assert b1[0, 13, 0] == 1          # blocks 1 and 2 tie: the lower wins
    assert b1[0, 8, 0] == 0
    assert b1[0, 3, 0] == -1 and b1[0, 4, 0] == 0
    r1 = oracle.select_routes(b1)
    assert r1.shape == (1, 14, 8)
    assert r1[0, 13].tolist() == [4, 5, 6, 7, 12, 13, -1, -1]
    assert r1[0, 8].tolist() == [0, 1, 2, 3, 8, -1, -1, -1]
    assert r1[0, 3].tolist() == [-1, -1, -1, -1, 0, 1, 2, 3]
    assert r1[0, 4].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]

    b2 = oracle.select_blocks(s, 2)
    assert b2[0, 13].tolist() == [1, 2]
    assert b2[0, 8].tolist() == [0, 1]            # a zero score still counts as visible
    assert b2[0, 5].tolist() == [0, -1]           # one visible block for two slots
    r2 = oracle.select_routes(b2)
    assert r2[0, 13].tolist() == [4, 5, 6, 7, 8, 9, 10, 11, 12, 13, -1, -1]
    assert r2[0, 5].tolist() == [0, 1, 2, 3, -1, -1, -1, -1, 4, 5, -1, -1]
    # top_k at least the visible count keeps every visible block
    b9 = oracle.select_blocks(s, 9)
    assert b9[0, 13, :4].tolist() == [0, 1, 2, -1]


def test_hand_document_metadata():
    # queries at positions 10..15; kbar rows (1,0), (0,1), (1,1), (2,0)
    K4 = np.array([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, 0.0]]])
    q = np.zeros((1, 6, 1, 2))
    q[0, 5, 0] = [1, 1]
    q[0, 0, 0] = [1, 0]     # dots 1, 0 with rows 0, 1
    q[0, 2, 0] = [0, 1]
    q[0, 4, 0] = [1, 1]
    start = np.array([[0, 8, 8, -1, 0, 20]], np.int32)   # the last starts after itself
    base = np.array([[0, 2, 2, 0, 3, 0]], np.int32)
    s = oracle.select_scores(q, K4, 0.5, q_offset=10, doc_start=start, blk_base=base)
    assert np.array_equal(s[0, 0], [0.5, 0.0, -INF, -INF])      # p 10, doc at 0: rows 0, 1
    assert np.isneginf(s[0, 1]).all()                            # p 11, doc at 8: no block yet
    assert np.array_equal(s[0, 2], [-INF, -INF, 0.5, -INF])     # p 12: block 0 is row 2
    assert np.isneginf(s[0, 3]).all()                            # padding query
    assert np.array_equal(s[0, 4], [-INF, -INF, -INF, 1.0])     # rows 3, 4, 5: only 3 exists
    assert np.isneginf(s[0, 5]).all()                            # padding: start past p
    vis, c = oracle.select_visible(1, 6, 4, 10, start, base)
    assert c[0].tolist() == [2, 0, 1, -1, 3, -1]
    b = oracle.select_blocks(s, 1, q_offset=10, doc_start=start, blk_base=base)
    assert b[0, :, 0].tolist() == [0, -1, 0, -1, 0, -1]
    r = oracle.select_routes(b, q_offset=10, doc_start=start)
    assert r[0].tolist() == [
        [0, 1, 2, 3, 8, 9, 10, -1],
        [-1, -1, -1, -1, 8, 9, 10, 11],
        [8, 9, 10, 11, 12, -1, -1, -1],
        [-1] * 8,
        [0, 1, 2, 3, 12, 13, 14, -1],
        [-1] * 8,
    ]


def _bf16(rng, shape, lo=-1.0, hi=1.0):
    return synth.bf16_bits(rng.uniform(lo, hi, shape).astype(np.float32))


def test_plus_minus_head_pairs_give_absolute_dots():
    rng = np.random.default_rng(5)
    B, Sq, m, d, NB = 2, 40, 3, 16, 9
    half = oracle.widen(_bf16(rng, (B, Sq, m, d)))
    q = np.concatenate([half, -half], axis=2)            # heads i and m + i opposite
    k = oracle.widen(_bf16(rng, (B, NB, d)))
    s = oracle.select_scores(q, k, 0.25, q_offset=3)
    want = 0.25 * np.abs(np.matmul(half, k.swapaxes(1, 2)[:, None])).sum(axis=2)
    fin = np.isfinite(s)
    assert np.allclose(s[fin], want[fin], rtol=1e-12, atol=0)
    # finite entries: rows below (q_offset + t) // 4
    cnt = np.minimum((3 + np.arange(Sq)) // 4, NB)
    assert np.array_equal(fin.sum(axis=2), np.broadcast_to(cnt, (B, Sq)))


def test_nonnegative_inputs_give_one_matrix_product():
    rng = np.random.default_rng(6)
    B, Sq, H, d, NB = 1, 64, 5, 8, 16
    q = oracle.widen(_bf16(rng, (B, Sq, H, d), 0.0, 1.0))
    k = oracle.widen(_bf16(rng, (B, NB, d), 0.0, 1.0))
    s = oracle.select_scores(q, k, 0.125)
    want = 0.125 * (q[0].sum(axis=1) @ k[0].T)           # [Sq, NB]
    fin = np.isfinite(s[0])
    assert np.allclose(s[0][fin], want[fin], rtol=1e-12, atol=0)


@pytest.mark.parametrize("ties", [False, True])
def test_top_k_against_stable_argsort(ties):
    rng = np.random.default_rng(7 + ties)
    B, Sq, NB, k = 2, 90, 24, 5
    scores = rng.integers(0, 4, (B, Sq, NB)).astype(np.float64) if ties else rng.random((B, Sq, NB))
    start = rng.integers(-1, 3, (B, Sq)).astype(np.int32)
    base = rng.integers(-2, 6, (B, Sq)).astype(np.int32)
    vis, _ = oracle.select_visible(B, Sq, NB, 0, start, base)
    scores = np.where(vis, scores, -np.inf)
    got = oracle.select_blocks(scores, k, 0, start, base)
    for b in range(B):
        for t in range(Sq):
            rows = np.nonzero(vis[b, t])[0]
            order = rows[np.argsort(-scores[b, t, rows], kind="stable")]
            want = np.sort(order[:k]) - base[b, t]
            assert got[b, t, :len(want)].tolist() == want.tolist()
            assert (got[b, t, len(want):] == -1).all()


@pytest.mark.parametrize("kind,seed", [("single", 11), ("docs", 12)])
def test_expansion_matches_synthetic_route_rows(kind, seed):
    """The synthetic generator writes route rows from (document start, chosen blocks,
    position); the oracle's expansion of the same block numbers must give them."""
    wl = synth.Workload("pin", 1, 300, 300, 12, 1, 256, 8, kind, seed, n_docs=5)
    inp = synth.make_inputs(wl, with_grad=False, record_blocks=True)
    rec = inp.info["row_blocks"]
    blocks = np.full((1, 300, 8), -1, np.int32)
    start = np.zeros((1, 300), np.int32)
    for i, (s0, chosen, c) in enumerate(rec):
        blocks[0, i, :len(chosen)] = chosen
        start[0, i] = s0
        assert c == (i - s0) // 4
    got = oracle.select_routes(blocks, 0, start)
    assert np.array_equal(got, inp.routes)
