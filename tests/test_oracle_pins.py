"""Pins of the FP64 oracle against facts fixed outside of it (CPU only).

Each test compares the oracle with something it does not share code with:
a hand derivation, a dense NumPy brute force, central finite differences,
torch's scaled_dot_product_attention (float64, CPU), closed forms and
invariants of the definition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dense_ref import dense_backward, dense_forward, dense_mask
from token_indexed_sparse_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, B=1, Sq=40, Skv=37, Hq=12, Hkv=1, W=11, D=16, causal=False, dtype=np.int32):
    c = synth.random_case(seed, B, Sq, Skv, Hq, Hkv, W, D=D, causal=causal, route_dtype=dtype)
    return c


def _problem(c, scale=0.37):
    return oracle.Problem(c.q, c.k, c.v, c.routes, scale, c.grad_out)


# ---------------------------------------------------------------- hand example
def test_hand_example():
    fx = json.load(open(os.path.join(GOLDEN, "hand_two_rows.json")))
    routes = np.array(fx["routes"], dtype=np.int32)
    P = oracle.Problem(np.array(fx["q"]), np.array(fx["k"]), np.array(fx["v"]), routes,
                       fx["scale"], np.array(fx["grad_out"]))
    out, lse = P.forward_full()
    np.testing.assert_allclose(out, np.array(fx["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(fx["lse"]), rtol=0, atol=1e-14)
    dq, dk, dv = P.backward_full()
    np.testing.assert_allclose(dq, np.array(fx["dq"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, np.array(fx["dk"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, np.array(fx["dv"]), rtol=0, atol=1e-14)
    # the stored numbers are the closed forms of the derivation
    e = math.e
    assert abs(fx["lse"][0][0][0] - math.log(e + 1)) < 1e-15
    assert abs(fx["dq"][0][0][0][1] - 2 * e / (e + 1) ** 2) < 1e-15


# ---------------------------------------------------------------- membership
@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_membership_matches_dense_scatter(dtype):
    c = _case(3, B=2, Sq=70, Skv=150, W=23, dtype=dtype)
    memb, has = oracle.membership(c.routes, 150)
    m = dense_mask(c.routes, 150)
    assert memb.shape == (2, 70, 256)
    assert np.array_equal(memb[:, :, :150].astype(bool), m)
    assert not memb[:, :, 150:].any()
    assert np.array_equal(has.astype(bool), m.any(-1))


def test_route_set_sorted_unique_and_int64_range():
    routes = np.array([[[5, 3, 5, -1, 2**32 + 3, 7, 3, np.iinfo(np.int64).min, 9]]], np.int64)
    assert list(oracle.route_set(routes, 9, 0)) == [3, 5, 7]
    assert list(oracle.route_set(routes, 10, 0)) == [3, 5, 7, 9]
    r32 = np.array([[[2**31 - 1, -2**31, 4, 4]]], np.int32)
    assert list(oracle.route_set(r32, 5, 0)) == [4]


# ---------------------------------------------------------------- tiles
def _tiles_numpy(memb, Sq, Skv, t=128):
    B = memb.shape[0]
    nqt, nkt = -(-Sq // t), -(-Skv // t)
    pad = np.zeros((B, nqt * t, nkt * t), np.int64)
    pad[:, :Sq, :Skv] = memb[:, :, :Skv]
    cnt = pad.reshape(B, nqt, t, nkt, t).sum((2, 4))
    return np.where(cnt == 0, 0, np.where(cnt == t * t, 2, 1)).astype(np.int32)


def _check_lists(T, kinds):
    B, nqt, nkt = kinds.shape
    for b in range(B):
        for r in range(nqt):
            for name, kd in (("p", 1), ("f", 2)):
                want = np.nonzero(kinds[b, r] == kd)[0]
                idx = T[f"fwd_{name}_idx"][b, r]
                assert T[f"fwd_{name}_cnt"][b, r] == len(want)
                assert np.array_equal(idx[: len(want)], want)
                assert (idx[len(want):] == -1).all()
        for t in range(nkt):
            for name, kd in (("p", 1), ("f", 2)):
                want = np.nonzero(kinds[b, :, t] == kd)[0]
                idx = T[f"rev_{name}_idx"][b, t]
                assert T[f"rev_{name}_cnt"][b, t] == len(want)
                assert np.array_equal(idx[: len(want)], want)
                assert (idx[len(want):] == -1).all()


def test_tiles_random_against_reshape_sum():
    rng = np.random.default_rng(0)
    B, Sq, Skv = 2, 300, 390
    memb = np.zeros((B, Sq, oracle.row_stride(Skv)), np.uint8)
    memb[:, :, :Skv] = rng.random((B, Sq, Skv)) < 0.02
    memb[:, 0:128, 128:256] = 1          # a full tile
    memb[:, 128:256, 0:128] = 0          # an absent tile
    memb[:, 256:300, 256:384] = 1        # ragged rows: never full
    T = oracle.tiles(memb, Skv)
    want = _tiles_numpy(memb, Sq, Skv)
    assert np.array_equal(T["kinds"], want)
    assert T["kinds"][0, 0, 1] == 2 and T["kinds"][0, 1, 0] == 0 and T["kinds"][0, 2, 2] == 1
    _check_lists(T, T["kinds"])


def test_tiles_special_routes():
    Sq = Skv = 256
    # all -1 -> every tile absent
    T = oracle.tiles(oracle.membership(np.full((1, Sq, 3), -1, np.int32), Skv)[0], Skv)
    assert (T["kinds"] == 0).all() and (T["fwd_p_cnt"] == 0).all() and (T["rev_f_idx"] == -1).all()
    # every key -> every tile full
    allk = np.broadcast_to(np.arange(Skv, dtype=np.int32), (1, Sq, Skv)).copy()
    T = oracle.tiles(oracle.membership(allk, Skv)[0], Skv)
    assert (T["kinds"] == 2).all()
    # complete causal routes -> lower tiles full, diagonal partial, upper absent
    causal = np.where(np.arange(Skv)[None, :] <= np.arange(Sq)[:, None], np.arange(Skv), -1)
    T = oracle.tiles(oracle.membership(causal[None].astype(np.int32), Skv)[0], Skv)
    assert T["kinds"][0].tolist() == [[1, 0], [2, 1]]
    # ragged edge tile holding every in-range key is still partial
    allk = np.broadcast_to(np.arange(200, dtype=np.int32), (1, 200, 200)).copy()
    T = oracle.tiles(oracle.membership(allk, 200)[0], 200)
    assert T["kinds"][0].tolist() == [[2, 1], [1, 1]]


def test_tiles_tiny_workload_closed_form():
    fx = json.load(open(os.path.join(GOLDEN, "tile_counts.json")))
    inp = synth.make_inputs(synth.WORKLOADS[1], with_grad=False)
    T = oracle.tiles(oracle.membership(inp.routes, 256)[0], 256)
    assert T["kinds"].tolist() == fx["tiny_s256_12q1kv"]["kinds"]


@pytest.mark.slow
@pytest.mark.parametrize("idx,name", [(4, "long_t32768_12q1kv"), (5, "cp_shard_q4096_kv32768_12q1kv")])
def test_tiles_large_workloads_closed_form(idx, name):
    fx = json.load(open(os.path.join(GOLDEN, "tile_counts.json")))[name]
    wl = synth.WORKLOADS[idx]
    rng = np.random.default_rng(wl.seed)
    routes, _ = synth.make_routes(wl, rng)
    T = oracle.tiles(oracle.membership(routes, wl.Skv)[0], wl.Skv)
    k = T["kinds"]
    assert [(k == 0).sum(), (k == 1).sum(), (k == 2).sum()] == [fx["absent"], fx["partial"], fx["full"]]


# ---------------------------------------------------------------- forward
@pytest.mark.parametrize("seed,B,Sq,Skv,Hq,Hkv,W,D", [
    (1, 1, 40, 37, 12, 1, 11, 16),
    (2, 2, 33, 50, 24, 2, 9, 8),
    (3, 1, 20, 20, 4, 2, 30, 256),
])
def test_forward_matches_dense_bruteforce(seed, B, Sq, Skv, Hq, Hkv, W, D):
    c = _case(seed, B, Sq, Skv, Hq, Hkv, W, D)
    P = _problem(c)
    out, lse = P.forward_full()
    m = dense_mask(c.routes, Skv)
    o2, l2 = dense_forward(P.q, P.k, P.v, m, P.scale)
    np.testing.assert_allclose(out, o2, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(l2))
    fin = np.isfinite(l2)
    np.testing.assert_allclose(lse[fin], l2[fin], rtol=1e-12, atol=1e-12)
    assert (np.isneginf(lse) == ~m.any(-1)[:, None, :]).all()


def test_forward_single_key_closed_form():
    c = _case(5, Sq=10, Skv=30, W=4, D=32)
    c.routes[:] = -1
    c.routes[0, :, 2] = np.arange(10) * 3
    P = _problem(c, scale=0.11)
    out, lse = P.forward_full()
    for i in range(10):
        j = 3 * i
        np.testing.assert_allclose(out[0, i], np.repeat(P.v[0, j], 12, 0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], 0.11 * P.q[0, i] @ P.k[0, j, 0], rtol=1e-13, atol=1e-15)


def test_forward_identical_keys_closed_form():
    c = _case(6, Sq=8, Skv=20, W=7, D=16)
    c.k[:] = c.k[:, :1]
    P = _problem(c, scale=0.5)
    out, lse = P.forward_full()
    for i in range(8):
        R = oracle.route_set(c.routes, 20, i)
        if len(R) == 0:
            assert (out[0, i] == 0).all() and np.isneginf(lse[0, :, i]).all()
            continue
        np.testing.assert_allclose(out[0, i], np.repeat(P.v[0, R].mean(0), 12, 0), atol=1e-13)
        s = 0.5 * P.q[0, i] @ P.k[0, 0, 0]
        np.testing.assert_allclose(lse[0, :, i], s + math.log(len(R)), rtol=1e-13)


def _sdpa(q, k, v, scale, causal):
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, G, 2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, G, 2)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_forward_equals_library_attention(causal):
    c = _case(7, B=2, Sq=24, Skv=24, Hq=24, Hkv=2, W=24, D=32)
    base = np.arange(24, dtype=np.int32)
    r = np.broadcast_to(base, (2, 24, 24)).copy()
    if causal:
        r = np.where(base[None, None, :] <= np.arange(24)[None, :, None], r, -1).astype(np.int32)
    rng = np.random.default_rng(1)
    r = np.take_along_axis(r, rng.permuted(np.tile(np.arange(24), (2, 24, 1)), axis=2), 2)
    P = oracle.Problem(c.q, c.k, c.v, r, 0.2)
    out, _ = P.forward_full()
    np.testing.assert_allclose(out, _sdpa(P.q, P.k, P.v, 0.2, causal), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("seed,B,Sq,Skv,Hq,Hkv,W,D", [
    (11, 1, 30, 41, 12, 1, 13, 16),
    (12, 2, 17, 23, 24, 2, 8, 8),
])
def test_backward_matches_dense_closed_form(seed, B, Sq, Skv, Hq, Hkv, W, D):
    c = _case(seed, B, Sq, Skv, Hq, Hkv, W, D)
    P = _problem(c)
    dq, dk, dv = P.backward_full()
    m = dense_mask(c.routes, Skv)
    dq2, dk2, dv2 = dense_backward(P.q, P.k, P.v, P.dout, m, P.scale)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("Hq", [2, 12])
def test_backward_finite_differences(Hq):
    rng = np.random.default_rng(100 + Hq)
    B, Sq, Skv, Hkv, D, W = 1, 12, 12, 1, 8, 7
    routes = rng.integers(-2, 14, size=(B, Sq, W)).astype(np.int32)   # dups, -1/-2, 12, 13
    routes[0, 3] = -1                                                 # an empty row
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Skv, Hkv, D))
    v = rng.standard_normal((B, Skv, Hkv, D))
    g = rng.standard_normal((B, Sq, Hq, D))
    scale = 0.7
    P = oracle.Problem(q, k, v, routes, scale, g)
    dq, dk, dv = P.backward_full()

    def loss(qq, kk, vv):
        o, _ = oracle.Problem(qq, kk, vv, routes, scale).forward_full()
        return float((o * g).sum())

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err < 1e-6, (name, err)
    assert (dq[0, 3] == 0).all()


def test_backward_sum_identities():
    c = _case(13, B=2, Sq=35, Skv=29, Hq=24, Hkv=2, W=10, D=16)
    P = _problem(c)
    dq, dk, dv = P.backward_full()
    # sum_j dS_ij = 0 for every (i, h)  =>  sum over keys of dK vanishes
    np.testing.assert_allclose(dk.sum(1), 0.0, atol=1e-10)
    # sum_j P_ij = 1 on non-empty rows  =>  sum over keys of dV = sum of dO over those rows
    m = dense_mask(c.routes, 29).any(-1)                       # [B, Sq]
    go = np.where(m[:, :, None, None], P.dout, 0.0)
    want = go.reshape(2, 35, 2, 12, 16).sum((1, 3))
    np.testing.assert_allclose(dv.sum(1), want, rtol=1e-11, atol=1e-11)


def test_backward_single_key_gives_zero_dq():
    c = _case(14, Sq=6, Skv=9, W=3, D=16)
    c.routes[:] = -1
    c.routes[0, :, 1] = [0, 2, 4, 6, 8, 8]
    dq, dk, dv = _problem(c).backward_full()
    assert np.abs(dq).max() < 1e-14
    assert np.abs(dk).max() < 1e-14


def test_backward_sampled_keys_and_rows_match_full():
    c = _case(15, B=2, Sq=40, Skv=33, Hq=24, Hkv=2, W=12, D=16)
    P = _problem(c)
    dq, dk, dv = P.backward_full()
    rows = np.array([0, 7, 41, 79], np.int64)
    dq_s = P.backward_dq(rows)
    np.testing.assert_allclose(dq_s, dq.reshape(-1, 24, 16)[rows], rtol=1e-13, atol=1e-13)
    keys = np.array([0, 5, 32, 33 + 4, 33 + 32], np.int64)
    dk_s, dv_s = P.backward_dkdv(keys)
    np.testing.assert_allclose(dk_s, dk.reshape(-1, 2, 16)[keys], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv_s, dv.reshape(-1, 2, 16)[keys], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariants
def _all_outputs(q, k, v, routes, g, scale=0.3):
    P = oracle.Problem(q, k, v, routes, scale, g)
    out, lse = P.forward_full()
    dq, dk, dv = P.backward_full()
    return out, lse, dq, dk, dv


def test_invariance_route_order_duplicates_and_invalid_ids():
    c = _case(21, B=1, Sq=30, Skv=40, W=12, D=16, dtype=np.int64)
    base = _all_outputs(c.q, c.k, c.v, c.routes, c.grad_out)
    rng = np.random.default_rng(5)
    perm = np.take_along_axis(c.routes, rng.permuted(np.tile(np.arange(12), (1, 30, 1)), axis=2), 2)
    dup = c.routes.copy()
    for i in range(30):
        valid = dup[0, i][(dup[0, i] >= 0) & (dup[0, i] < 40)]
        pad = dup[0, i] == -1
        if len(valid):
            dup[0, i, pad] = valid[0]
    bad = c.routes.copy()
    for val in (40, 47, -5, 2**32 + 5, np.iinfo(np.int64).min):
        b2 = bad.copy()
        b2[b2 == -1] = val
        for x, y in zip(base, _all_outputs(c.q, c.k, c.v, b2, c.grad_out)):
            assert np.array_equal(x, y)
    for r in (perm, dup):
        for x, y in zip(base, _all_outputs(c.q, c.k, c.v, r, c.grad_out)):
            assert np.array_equal(x, y)


def test_padding_rows_and_unselected_nan():
    c = _case(22, B=1, Sq=20, Skv=30, W=6, D=16)
    c.routes[0, 4] = -1
    c.routes[c.routes >= 25] = 1                     # keys 25.. selected by nobody
    q = oracle.widen(c.q)
    k = oracle.widen(c.k)
    v = oracle.widen(c.v)
    q[0, 4] = np.nan                                  # Q of a padding row is irrelevant
    k[0, 25:] = np.nan
    v[0, 26:] = np.inf
    out, lse, dq, dk, dv = _all_outputs(q, k, v, c.routes, c.grad_out)
    assert np.isfinite(out).all() and np.isfinite(dq).all()
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    assert (out[0, 4] == 0).all() and not np.signbit(out[0, 4]).any()
    assert np.isneginf(lse[0, :, 4]).all()
    assert (dq[0, 4] == 0).all()
    assert (dk[0, 25:] == 0).all() and (dv[0, 25:] == 0).all()


def test_backward_on_saved_state_matches_dense_closed_form():
    # The backward equations take the saved O and LSE as inputs (a GPU run feeds
    # its out_fp32 and lse). With perturbed saved values the oracle must follow
    # the same closed form as the dense NumPy backward fed the same values, and
    # differ from its own-forward result (the saved values are really used).
    c = _case(16, B=2, Sq=33, Skv=27, Hq=24, Hkv=2, W=11, D=16)
    P = _problem(c)
    own = P.backward_full()
    o, lse = P.forward_full()
    rng = np.random.default_rng(5)
    o2 = o + 1e-2 * rng.standard_normal(o.shape)
    lse2 = np.where(np.isfinite(lse), lse + 1e-2 * rng.standard_normal(lse.shape), lse)
    P.use_saved(o2, lse2)
    got = P.backward_full()
    m = dense_mask(c.routes, 27)
    want = dense_backward(P.q, P.k, P.v, P.dout, m, P.scale, out=o2, lse=lse2)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
    rows = np.array([0, 5, 40, 65], np.int64)
    np.testing.assert_allclose(P.backward_dq(rows), got[0].reshape(-1, 24, 16)[rows],
                               rtol=1e-12, atol=1e-12)
    keys = np.array([0, 3, 30, 53], np.int64)
    dk, dv = P.backward_dkdv(keys)
    np.testing.assert_allclose(dk, got[1].reshape(-1, 2, 16)[keys], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv, got[2].reshape(-1, 2, 16)[keys], rtol=1e-11, atol=1e-11)
    assert np.abs(got[0] - own[0]).max() > 1e-4
    P.use_saved(None, None)
    again = P.backward_full()
    for a, b in zip(again, own):
        np.testing.assert_array_equal(a, b)


def test_all_outputs_pass_matches_separate_calls():
    c = _case(17, B=2, Sq=31, Skv=40, Hq=24, Hkv=2, W=9, D=16)
    P = _problem(c)
    o, lse, dq, dk, dv = P.all_outputs()
    o2, lse2 = P.forward_full()
    dq2, dk2, dv2 = P.backward_full()
    for a, b in ((o, o2), (lse, lse2), (dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_array_equal(a, b)
    m = dense_mask(c.routes, 40)
    o3, lse3 = dense_forward(P.q, P.k, P.v, m, P.scale)
    np.testing.assert_allclose(o, o3, rtol=1e-12, atol=1e-12)
