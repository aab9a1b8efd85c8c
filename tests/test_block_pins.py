"""Pins of the oracle's block-bitmap selection (the Miles lookup of the cuDNN
Frontend QSA page, section "Selection and components"): for packed tokens,
key j is allowed for query t iff lo[t] <= j <= hi[t], 0 <= b < NB and
sel_blocks[t, b] != 0, with b = blk_base[t] + floor((j - tok_base[t]) / 4).

The hand cases are worked out from that statement by hand and typed in as
sets. The workload cases build the bitmap from the block numbers the route
generator drew (never from route values or the lookup), so the oracle's lookup
must reproduce the route membership of the same draw: a wrong rounding of the
division, a dropped base or bound, or a block numbering that does not restart
per document fails them.
"""
import numpy as np
import pytest

import oracle
from token_indexed_sparse_amd import synth

# Ten packed tokens: sequence A = tokens 0..5 (blocks 0 = 0..3, 1 = 4..5),
# sequence B = tokens 6..9 (block 2 = 6..9), so B's first token is not a
# multiple of four and its numbering restarts at block 2.
HAND_T, HAND_NB = 10, 3
HAND_ROWS = {
    # t: (lo, hi, blk_base, tok_base, selected blocks, allowed keys)
    0: (0, 0, 0, 0, [0], {0}),
    1: (5, 3, 0, 0, [0, 1, 2], set()),             # lo > hi: empty
    2: (1, 2, 0, 0, [0, 1, 2], {1, 2}),            # the bounds cut the block
    3: (0, 3, 0, 0, [0], {0, 1, 2, 3}),
    4: (0, 4, -1, 0, [0, 1], {4}),                 # keys 0..3 map to block -1
    5: (0, 5, 0, 0, [1, 2], {4, 5}),               # block 2 lies past hi
    6: (6, 9, 2, 2, [0, 1, 2], set()),             # keys map to block 3 = NB
    7: (6, 7, 2, 6, [0, 1, 2], {6, 7}),            # blocks 0, 1 unreachable
    8: (0, 9, 2, 6, [1, 2], {2, 3, 4, 5, 6, 7, 8, 9}),  # floor: keys 0, 1 -> block 0
    9: (6, 9, 2, 6, [0], set()),
}


def _hand():
    sel = np.zeros((HAND_T, HAND_NB), np.uint8)
    meta = np.zeros((4, HAND_T), np.int32)
    for t, (lo, hi, bb, tb, blocks, _) in HAND_ROWS.items():
        sel[t, blocks] = 1
        meta[:, t] = (lo, hi, bb, tb)
    return sel, meta


def test_hand_cases():
    sel, (lo, hi, bb, tb) = _hand()
    memb, has = oracle.block_membership(sel, lo, hi, bb, tb)
    assert memb.shape == (1, HAND_T, 128)
    assert not memb[0, :, HAND_T:].any()  # padding columns past the last token
    for t, row in HAND_ROWS.items():
        got = set(np.nonzero(memb[0, t])[0].tolist())
        assert got == row[5], (t, got, row[5])
        assert has[0, t] == (1 if row[5] else 0)


def test_nonzero_bytes_select_and_routes_round_trip():
    sel, (lo, hi, bb, tb) = _hand()
    memb, _ = oracle.block_membership(sel * 7, lo, hi, bb, tb)  # any nonzero byte selects
    ref, _ = oracle.block_membership(sel, lo, hi, bb, tb)
    assert np.array_equal(memb, ref)
    routes = oracle.routes_from_membership(memb, HAND_T)
    again, _ = oracle.membership(routes, HAND_T)
    assert np.array_equal(again, memb)


def _docs_workload():
    # five documents in 300 tokens; the seed gives cuts that are not multiples of 4
    return synth.Workload("docs_300", 1, 300, 300, 12, 1, 256, 8, "docs", 7, n_docs=5)


@pytest.mark.parametrize("wl", [synth.WORKLOADS[1], _docs_workload(), synth.WORKLOADS[2],
                                synth.WORKLOADS[3]], ids=lambda w: w.name)
def test_bitmap_of_drawn_blocks_matches_route_membership(wl):
    inp = synth.make_inputs(wl, record_blocks=True)
    # same draws with and without the record
    assert np.array_equal(inp.routes, synth.make_inputs(wl).routes)
    bi = synth.block_inputs(inp)
    if wl.kind == "docs":
        starts = inp.info["doc_starts"]
        assert any(int(s) % 4 for s in starts), "need a document start off the 4-grid"
    memb, has = oracle.block_membership(bi.sel_blocks, bi.lo, bi.hi, bi.blk_base, bi.tok_base)
    ref, ref_has = oracle.membership(bi.routes, bi.T)
    assert np.array_equal(memb, ref)
    assert np.array_equal(has, ref_has)
    # the block spans describe the same numbering the rows use
    for t in range(0, bi.T, max(1, bi.T // 64)):
        if bi.hi[t] < bi.lo[t]:
            continue
        b_own = bi.blk_base[t] + (t - bi.tok_base[t]) // 4
        assert bi.block_first[b_own] <= t <= bi.block_last[b_own]
