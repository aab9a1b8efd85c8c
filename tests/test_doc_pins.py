"""Pins of the oracle's document-causal selection ("fa4" page,
`document_causal_fa4_attention`): query i of batch row b, at global position
p = q_global_start + i, sees key j iff q_doc[b, i] != 0, kv_doc[b, j] == q_doc[b, i]
and j <= p.

The hand cases are worked out from that statement and typed in as matrices. The
workload cases build route rows listing, for every query, the keys from its
document's first token to its own position (numpy ranges from the drawn document
cuts, never the oracle's test), and the oracle's document-causal membership must
equal their route membership: a dropped causal bound, an off-by-one at the
query's own position, a lost shard offset or an attended padding token fails them.
"""
import numpy as np
import pytest

import oracle
from token_indexed_sparse_amd import synth

Q_DOC = np.array([[1, 1, 2, 2, 0, 2]], np.int32)
KV_DOC = np.array([[1, 1, 2, 2, 2, 2, 3]], np.int32)
# q_global_start = 0: query i sits at key position i
HAND_0 = np.array([
    [1, 0, 0, 0, 0, 0, 0],
    [1, 1, 0, 0, 0, 0, 0],
    [0, 0, 1, 0, 0, 0, 0],
    [0, 0, 1, 1, 0, 0, 0],
    [0, 0, 0, 0, 0, 0, 0],   # padding query
    [0, 0, 1, 1, 1, 1, 0],   # document 2 up to position 5; key 6 is document 3
], np.uint8)
# q_global_start = 1: every query one position later
HAND_1 = np.array([
    [1, 1, 0, 0, 0, 0, 0],
    [1, 1, 0, 0, 0, 0, 0],   # document 1 has only keys 0, 1
    [0, 0, 1, 1, 0, 0, 0],
    [0, 0, 1, 1, 1, 0, 0],
    [0, 0, 0, 0, 0, 0, 0],
    [0, 0, 1, 1, 1, 1, 0],   # position 6 is document 3
], np.uint8)


@pytest.mark.parametrize("start,want", [(0, HAND_0), (1, HAND_1)])
def test_hand_cases(start, want):
    memb, has = oracle.doc_membership(Q_DOC, KV_DOC, start)
    assert memb.shape == (1, 6, 128)
    assert np.array_equal(memb[0, :, :7], want)
    assert not memb[0, :, 7:].any()
    assert np.array_equal(has[0], want.any(axis=1).astype(np.uint8))


def _doc_ids(starts: np.ndarray, T: int) -> np.ndarray:
    ids = np.zeros(T, np.int32)
    for n, s0 in enumerate(starts):
        ids[s0:] = n + 1
    return ids


def _causal_routes(starts: np.ndarray, positions: np.ndarray, T: int) -> np.ndarray:
    """Route rows listing keys doc_start(p) .. p for each query position p."""
    bounds = np.concatenate([starts, [T]])
    rows = []
    for p in positions:
        d = np.searchsorted(bounds, p, side="right") - 1
        rows.append(np.arange(bounds[d], p + 1))
    W = max(len(r) for r in rows)
    out = np.full((1, len(rows), W), -1, np.int32)
    for i, r in enumerate(rows):
        out[0, i, :len(r)] = r
    return out


@pytest.mark.parametrize("T,n_docs,seed", [(300, 5, 7), (2048, 4, 2)])
def test_documents_match_route_rows(T, n_docs, seed):
    wl = synth.Workload("docs", 1, T, T, 12, 1, 256, 8, "docs", seed, n_docs=n_docs)
    starts = synth.make_inputs(wl, with_grad=False).info["doc_starts"].astype(np.int64)
    ids = _doc_ids(starts, T)[None]
    memb, has = oracle.doc_membership(ids, ids, 0)
    ref, ref_has = oracle.membership(_causal_routes(starts, np.arange(T), T), T)
    assert np.array_equal(memb, ref)
    assert np.array_equal(has, ref_has)
    # a contiguous shard of the last quarter of the queries against all keys
    q0 = 3 * T // 4
    memb_s, _ = oracle.doc_membership(ids[:, q0:], ids, q0)
    ref_s, _ = oracle.membership(_causal_routes(starts, np.arange(q0, T), T), T)
    assert np.array_equal(memb_s, ref_s)


def test_padding_tokens():
    rng = np.random.default_rng(3)
    T = 257
    ids = rng.integers(0, 4, (2, T)).astype(np.int32)  # runs of any layout, with padding
    memb, has = oracle.doc_membership(ids, ids, 0)
    j = np.arange(T)
    for b in range(2):
        for i in range(T):
            want = (ids[b, i] != 0) & (ids[b] == ids[b, i]) & (j <= i)
            assert np.array_equal(memb[b, i, :T].astype(bool), want)
    assert not memb[ids == 0].any()          # padding queries attend to nothing
    assert not memb[:, :, :T][np.broadcast_to((ids == 0)[:, None, :], (2, T, T))].any()
