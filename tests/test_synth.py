"""The seeded workload generators produce the route structure they promise (CPU only)."""
import numpy as np
import pytest

from token_indexed_sparse_amd import synth


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, np.inf, 1e-40], np.float32)
    b = synth.bf16_bits(x)
    back = synth.bf16_to_f32(b)
    assert back.tolist()[:5] == [1.0, 1.0, 1.0 + 4 * 2**-8, 1.0, -2.5]
    assert np.isinf(back[5])
    assert np.isnan(synth.bf16_to_f32(synth.bf16_bits(np.array([np.nan], np.float32))))[0]


def _check_row(row, n_max, doc_start, pos):
    c = (pos - doc_start) // 4
    own = row[4 * n_max:]
    want_own = list(range(doc_start + 4 * c, pos + 1))
    assert own[: len(want_own)].tolist() == want_own
    assert (own[len(want_own):] == -1).all()
    body = row[: 4 * n_max].reshape(n_max, 4)
    used = body[body[:, 0] >= 0]
    assert (body[body[:, 0] < 0] == -1).all()
    blocks = (used[:, 0] - doc_start) // 4
    assert ((used - used[:, :1]) == np.arange(4)).all()
    assert ((used[:, 0] - doc_start) % 4 == 0).all()
    assert (np.diff(blocks) > 0).all() and (blocks < c).all() and (blocks >= 0).all()
    return blocks, c


def test_tiny_workload_structure_and_determinism():
    wl = synth.WORKLOADS[1]
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    assert a.routes.shape == (1, 256, 36) and a.routes.dtype == np.int32
    assert np.array_equal(a.routes, b.routes) and np.array_equal(a.q, b.q)
    assert a.q.shape == (1, 256, 12, 256) and a.k.shape == (1, 256, 1, 256)
    for p in range(256):
        blocks, c = _check_row(a.routes[0, p], 8, 0, p)
        assert len(blocks) == min(8, c)


def test_docs_workload_structure():
    wl = synth.WORKLOADS[2]
    rng = np.random.default_rng(wl.seed)
    routes, info = synth.make_routes(wl, rng)
    starts = info["doc_starts"]
    assert routes.shape == (1, 8192, 260) and len(starts) == 4 and starts[0] == 0
    for p in range(0, 8192, 7):
        s = int(starts[np.searchsorted(starts, p, side="right") - 1])
        blocks, c = _check_row(routes[0, p], 64, s, p)
        assert len(blocks) == min(64, c)


def test_padded_workload_structure():
    wl = synth.WORKLOADS[3]
    rng = np.random.default_rng(wl.seed)
    routes, info = synth.make_routes(wl, rng)
    L = info["lengths"]
    assert routes.shape == (4, 4096, 260)
    assert ((L >= 1024) & (L <= 4096)).all()
    for b in range(4):
        assert (routes[b, L[b]:] == -1).all()
        for p in range(0, int(L[b]), 13):
            blocks, c = _check_row(routes[b, p], 64, 0, p)
            assert len(blocks) == min(64, c)


@pytest.mark.slow
def test_long_and_shard_workload_structure():
    wl = synth.WORKLOADS[4]
    routes, _ = synth.make_routes(wl, np.random.default_rng(wl.seed))
    assert routes.shape == (1, 32768, 2052)
    for p in list(range(0, 32768, 997)) + [2047, 2048, 32767]:
        blocks, c = _check_row(routes[0, p], 512, 0, p)
        assert len(blocks) == min(c, 512)
        recent = np.arange(max(0, c - 256), c)
        assert np.isin(recent, blocks).all()
    wl = synth.WORKLOADS[5]
    routes, _ = synth.make_routes(wl, np.random.default_rng(wl.seed))
    assert routes.shape == (1, 4096, 1028)
    for i in range(0, 4096, 331):
        blocks, c = _check_row(routes[0, i], 256, 0, 28672 + i)
        assert len(blocks) == 256


def test_random_case_has_padding_duplicates_and_invalid():
    c = synth.random_case(0, 2, 50, 40, 12, 1, 16, route_dtype=np.int64)
    r = c.routes
    assert (r == -1).any() and (r >= 40).any() and (r < -1).any() and (r > 2**32).any()
    dups = sum(len(x[(x >= 0) & (x < 40)]) - len(np.unique(x[(x >= 0) & (x < 40)]))
               for x in r.reshape(-1, 16))
    assert dups > 0
    assert ((r == -1).all(-1)).sum() >= 2


def test_tiled_cases_have_full_and_partial_tiles():
    import oracle
    for kw, want_partial in ((dict(seed=51, B=1, Sq=384, Skv=384, Hq=12, Hkv=1, p_full=0.5,
                                   extra=30), True),
                             (dict(seed=52, B=2, Sq=300, Skv=520, Hq=24, Hkv=2, p_full=0.6,
                                   extra=10, bare_rows=True), True),
                             (dict(seed=53, B=1, Sq=384, Skv=384, Hq=12, Hkv=1, causal=True,
                                   extra=0), True),
                             (dict(seed=55, B=1, Sq=256, Skv=256, Hq=12, Hkv=1, all_keys=True,
                                   extra=0), False)):
        inp = synth.tiled_case(**kw)
        memb, _ = oracle.membership(inp.routes, kw["Skv"])
        kinds = oracle.tiles(memb, kw["Skv"])["kinds"]
        assert (kinds == 2).any(), kw
        assert ((kinds == 1).any()) == want_partial, kw
        # route slots hold a duplicate and an out-of-range value on every row
        r = inp.routes
        assert ((r == kw["Skv"] + 3).sum(-1) == 1).all()
    # causal-complete: full strictly below the diagonal, partial on it
    inp = synth.tiled_case(53, 1, 384, 384, 12, 1, causal=True, extra=0)
    memb, _ = oracle.membership(inp.routes, 384)
    kinds = oracle.tiles(memb, 384)["kinds"][0]
    assert (kinds == np.array([[1, 0, 0], [2, 1, 0], [2, 2, 1]])).all()
    # bare rows: odd query tiles of batch 0 select only whole tiles
    inp = synth.tiled_case(52, 2, 300, 520, 24, 2, p_full=0.6, extra=10, bare_rows=True)
    for row in inp.routes[0, 128:256]:
        keys = np.unique(row[(row >= 0) & (row < 520)])
        for t in np.unique(keys // 128):
            assert np.isin(np.arange(128 * t, min(128 * t + 128, 520)), keys).all()


def test_loud_last_case_forces_both_rescale_paths():
    """The loud-last tiled case has rows whose later keys score far above the
    first ones: in the dense pass (full tiles after the first, above the
    hand-over and the first 32 keys by more than 2^64) and in the gathered
    pass (partial keys after the first 16, in ascending key order). Scores are
    taken in log2 units, exactly as the kernels compare them."""
    Sq, Skv = 384, 512
    inp = synth.tiled_case(seed=56, B=1, Sq=Sq, Skv=Skv, Hq=12, Hkv=1, p_full=0.6, extra=20,
                           loud_keys=48.0, loud_last=True)
    q = synth.bf16_to_f32(inp.q)[0].astype(np.float64)
    k = synth.bf16_to_f32(inp.k)[0, :, 0].astype(np.float64)
    memb = np.zeros((Sq, Skv), bool)
    for i in range(Sq):
        v = inp.routes[0, i]
        memb[i, v[(v >= 0) & (v < Skv)]] = True
    full = memb.reshape(Sq // 128, 128, Skv // 128, 128).sum(axis=(1, 3)) == 128 * 128
    c = 0.0625 / np.log(2.0)
    dense_raise = gathered_restart = 0
    for i in range(Sq):
        s = q[i] @ k.T * c
        ft = np.nonzero(full[i // 128])[0]
        part = memb[i].copy()
        for t in ft:
            part[128 * t:128 * t + 128] = False
        if len(ft) >= 2:
            m_hand = s[:, part].max(axis=1) if part.any() else np.full(12, -np.inf)
            ref = np.maximum(m_hand, s[:, 128 * ft[0]:128 * ft[0] + 32].max(axis=1))
            later = np.concatenate([s[:, 128 * t:128 * t + 128] for t in ft], axis=1).max(axis=1)
            dense_raise += int((later > ref + 64).any())
        keys = np.nonzero(part)[0]
        if len(keys) > 16:
            gathered_restart += int((s[:, keys].max(axis=1) > s[:, keys[:16]].max(axis=1) + 64).any())
    assert dense_raise > 0 and gathered_restart > 0, (dense_raise, gathered_restart)
