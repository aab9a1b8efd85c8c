"""HIP path vs the FP64 oracle on the same seeded inputs (needs an MI355X).

Integer tables (membership, tile kinds, tile lists, per-row key lists) must
match bit-exactly. Floating outputs must satisfy |x - ref| <= tol + tol*|ref|
elementwise, with tol = 1e-3 for out_fp32 and lse and 2e-2 for the bf16
tensors out, dq, dk, dv; -inf LSE must match exactly. Small cases compare every
element; the full-size workloads compare sampled rows and keys that the oracle
computes one by one, plus properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL_BF16, TOL_FP32, DeviceRun, bf16_bits_of, check_close,
                      check_preprocess_exact, log, to_np)
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _full_compare(inp, scale, run=None):
    run = run or DeviceRun(inp, scale)
    P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, scale, inp.grad_out)
    o_ref, l_ref = P.forward_full()
    check_close("out_fp32", to_np(run.out32), o_ref, TOL_FP32)
    check_close("lse", to_np(run.lse), l_ref, TOL_FP32)
    check_close("out", to_np(run.out), o_ref, TOL_BF16)
    dq_ref, dk_ref, dv_ref = P.backward_full()
    check_close("dq", to_np(run.dq), dq_ref, TOL_BF16)
    check_close("dk", to_np(run.dk), dk_ref, TOL_BF16)
    check_close("dv", to_np(run.dv), dv_ref, TOL_BF16)
    # out is the bf16 rounding of the same kernel's out_fp32
    from token_indexed_sparse_amd.synth import bf16_bits
    assert np.array_equal(bf16_bits_of(run.out), bf16_bits(to_np(run.out32).astype(np.float32)))
    return run


# Small cases: several tiles, ragged tails, padding, duplicates, invalid IDs.
SMALL = [
    dict(seed=31, B=1, Sq=300, Skv=333, Hq=12, Hkv=1, W=40),
    dict(seed=32, B=2, Sq=129, Skv=260, Hq=24, Hkv=2, W=70),
    dict(seed=33, B=1, Sq=64, Skv=1000, Hq=12, Hkv=1, W=300),
    dict(seed=34, B=3, Sq=17, Skv=5, Hq=12, Hkv=1, W=3),
    dict(seed=35, B=1, Sq=200, Skv=200, Hq=12, Hkv=1, W=200, causal=True),
    # more query rows than one dK/dV query-range phase holds: accumulators carry over
    dict(seed=36, B=2, Sq=2300, Skv=200, Hq=24, Hkv=2, W=10),
    # rows too wide for the row's key list to be staged in LDS (over 64 KB):
    # the preprocessing writes it straight from its bitmap
    dict(seed=37, B=1, Sq=40, Skv=3000, Hq=12, Hkv=1, W=17000),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"seed{c['seed']}")
def test_small_cases_full_parity(case):
    log(f"case {case}")
    inp = synth.random_case(**case)
    run = DeviceRun(inp, 0.0625)
    check_preprocess_exact(inp.routes, case["Skv"], run.routes)
    _full_compare(inp, 0.0625, run)


# Full 128 x 128 tiles (the dense path) next to gathered keys: the hand-over
# between the two forward passes, rows with no gathered keys, causal-complete
# and all-full tile rows, edge tiles that are chosen whole but cannot be full,
# moderately large scores in the first full key tile (seed 54), and very large
# scores in the last one (seed 56), which make the dense pass redo its tiles
# with a raised reference maximum and the gathered pass restart rows (a CPU
# test checks that the case does force both).
TILED = [
    dict(seed=51, B=1, Sq=384, Skv=384, Hq=12, Hkv=1, p_full=0.5, extra=30),
    dict(seed=52, B=2, Sq=300, Skv=520, Hq=24, Hkv=2, p_full=0.6, extra=10, bare_rows=True),
    dict(seed=53, B=1, Sq=384, Skv=384, Hq=12, Hkv=1, causal=True, extra=0),
    dict(seed=54, B=1, Sq=256, Skv=384, Hq=12, Hkv=1, p_full=0.5, extra=20, loud_keys=8.0),
    dict(seed=55, B=1, Sq=256, Skv=256, Hq=12, Hkv=1, all_keys=True, extra=0),
    dict(seed=56, B=1, Sq=384, Skv=512, Hq=12, Hkv=1, p_full=0.6, extra=20, loud_keys=48.0,
         loud_last=True),
]


@pytest.mark.parametrize("case", TILED, ids=lambda c: f"seed{c['seed']}")
def test_full_tile_cases_parity(case):
    log(f"case {case}")
    inp = synth.tiled_case(**case)
    run = DeviceRun(inp, 0.0625)
    check_preprocess_exact(inp.routes, case["Skv"], run.routes)
    _full_compare(inp, 0.0625, run)


def test_int64_routes_huge_values_match_int32():
    inp = synth.random_case(41, 1, 150, 140, 12, 1, 30, route_dtype=np.int64)
    log("int64 routes with values beyond 2^31")
    run = DeviceRun(inp, 0.1)
    check_preprocess_exact(inp.routes, 140, run.routes)
    _full_compare(inp, 0.1, run)
    r32 = np.where((inp.routes >= 0) & (inp.routes < 140), inp.routes, -1).astype(np.int32)
    run32 = DeviceRun(inp, 0.1, routes=r32)
    for a, b in ((run.out32, run32.out32), (run.lse, run32.lse), (run.dq, run32.dq),
                 (run.dk, run32.dk), (run.dv, run32.dv)):
        assert torch.equal(a, b)


def test_tiny_workload_full_parity():
    wl = synth.WORKLOADS[1]
    log(f"workload {wl.name}")
    inp = synth.make_inputs(wl)
    run = DeviceRun(inp, wl.scale)
    check_preprocess_exact(inp.routes, wl.Skv, run.routes)
    _full_compare(inp, wl.scale, run)


def _sample_rows(wl, inp, rng, n=160):
    """At least 256 flat rows: the first and last rows, every 128-row tile boundary
    (rows 128t - 1, 128t), document starts and valid-length edges, and random rows."""
    rows = set(range(3)) | set(range(wl.Sq - 3, wl.Sq))
    for t in range(1, -(-wl.Sq // 128)):
        rows |= {128 * t - 1, 128 * t}
    rows = set(sorted(rows)[:96]) | set(range(wl.Sq - 3, wl.Sq))
    rows |= set(int(x) for x in rng.choice(wl.Sq, n, replace=False))
    while len(rows) < 256:
        rows.add(int(rng.integers(0, wl.Sq)))
    for s in inp.info.get("doc_starts", []):
        rows |= {int(s), min(int(s) + 5, wl.Sq - 1)}
    flat = []
    for b in range(wl.B):
        extra = set()
        if "lengths" in inp.info:
            L = int(inp.info["lengths"][b])
            extra = {L - 1, min(L, wl.Sq - 1), min(L + 1, wl.Sq - 1)}
        flat += [b * wl.Sq + r for r in sorted(rows | extra)]
    return np.array(sorted(set(flat)), np.int64)


def _sample_keys(wl, rng, n=24):
    """At least 64 flat keys: keys 0..15, both sides of every key-tile boundary
    that is a power-of-two multiple of 128, the last keys, and random keys."""
    keys = set(range(16)) | set(range(wl.Skv - 4, wl.Skv))
    t = 128
    while t < wl.Skv:
        keys |= {t - 1, t}
        t *= 2
    keys |= set(int(x) for x in rng.choice(wl.Skv, n, replace=False))
    while len(keys) < 64:
        keys.add(int(rng.integers(0, wl.Skv)))
    flat = []
    for b in range(wl.B):
        flat += [b * wl.Skv + k for k in sorted(keys)]
    return np.array(flat, np.int64)


def _check_all(run, refs, wl, label=""):
    o_ref, l_ref, dq_ref, dk_ref, dv_ref = refs
    check_close(f"{label}out_fp32 (all rows)", to_np(run.out32), o_ref, TOL_FP32)
    check_close(f"{label}lse (all rows)", to_np(run.lse), l_ref, TOL_FP32)
    check_close(f"{label}out (all rows)", to_np(run.out), o_ref, TOL_BF16)
    check_close(f"{label}dq (all rows)", to_np(run.dq), dq_ref, TOL_BF16)
    check_close(f"{label}dk (all keys)", to_np(run.dk), dk_ref, TOL_BF16)
    check_close(f"{label}dv (all keys)", to_np(run.dv), dv_ref, TOL_BF16)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_workload_parity(idx):
    """Every output element of the full-size workload against the oracle (one
    pass over all rows), then the oracle's backward fed the GPU's own out_fp32
    and lse on sampled rows and keys, which isolates the backward's error."""
    wl = synth.WORKLOADS[idx]
    log(f"workload {wl.name}: generating")
    inp = synth.make_inputs(wl)
    run = DeviceRun(inp, wl.scale)
    log("  preprocess check")
    check_preprocess_exact(inp.routes, wl.Skv, run.routes)
    P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, wl.scale, inp.grad_out)
    log(f"  oracle: all outputs ({oracle.num_threads()} threads)")
    _check_all(run, P.all_outputs(), wl)
    # backward on the GPU's saved state
    rng = np.random.default_rng(100 + idx)
    rows = _sample_rows(wl, inp, rng)
    keys = _sample_keys(wl, rng)
    assert len(rows) >= 256 and len(keys) >= 64
    P.use_saved(to_np(run.out32), to_np(run.lse))
    log(f"  oracle on the GPU's out_fp32 and lse: dq of {len(rows)} rows, dk/dv of "
        f"{len(keys)} keys")
    dq_s = P.backward_dq(rows)
    check_close("dq[rows] (saved state)", to_np(run.dq).reshape(-1, wl.Hq, wl.D)[rows], dq_s,
                TOL_BF16)
    dk_s, dv_s = P.backward_dkdv(keys)
    check_close("dk[keys] (saved state)", to_np(run.dk).reshape(-1, wl.Hkv, wl.D)[keys], dk_s,
                TOL_BF16)
    check_close("dv[keys] (saved state)", to_np(run.dv).reshape(-1, wl.Hkv, wl.D)[keys], dv_s,
                TOL_BF16)
    # properties at full size: empty rows are exactly zero with -inf lse
    has = (inp.routes >= 0).any(-1)
    empty = ~has
    if empty.any():
        o = to_np(run.out32)[empty]
        assert (o == 0).all() and not np.signbit(o).any()
        assert (to_np(run.dq)[empty] == 0).all()
        assert np.isneginf(to_np(run.lse).transpose(0, 2, 1)[empty]).all()


@pytest.mark.timeout(600)
def test_rotated_walks_with_restarts_and_redo():
    # 16384 query rows (eight per resident wave slot of a 256-CU device), so the
    # default mode rotates the gathered walks, with very large scores in the last
    # chosen key tile: rows whose walk starts mid-list meet the large scores
    # after smaller ones and restart, and the dense forward redoes its tiles.
    # Both modes against the oracle, and against each other.
    case = dict(seed=57, B=1, Sq=16384, Skv=512, Hq=12, Hkv=1, p_full=0.6, extra=20,
                loud_keys=48.0, loud_last=True)
    log(f"case {case}")
    inp = synth.tiled_case(**case)
    a = DeviceRun(inp, 0.0625, deterministic=True)
    b = DeviceRun(inp, 0.0625)
    P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, 0.0625, inp.grad_out)
    refs = P.all_outputs()
    wl = inp.wl
    _check_all(a, refs, wl, "deterministic ")
    _check_all(b, refs, wl, "default ")
    for name, x, y in (("out_fp32", a.out32, b.out32), ("lse", a.lse, b.lse)):
        x = x.double()
        y = y.double()
        fin = torch.isfinite(x)
        assert torch.equal(fin, torch.isfinite(y)) and torch.equal(x[~fin], y[~fin]), name
        err = ((x - y)[fin].abs() / (1e-4 + 1e-4 * x[fin].abs())).max().item()
        log(f"  {name}: max |default - deterministic| / (1e-4 + 1e-4 |x|) = {err:.3f}")
        assert err <= 1.0, name


def test_route_order_duplicates_invalid_ids_bitwise():
    inp = synth.random_case(51, 1, 260, 300, 12, 1, 48)
    base = DeviceRun(inp, 0.0625, deterministic=True)
    rng = np.random.default_rng(9)
    perm = np.take_along_axis(inp.routes,
                              rng.permuted(np.tile(np.arange(48), (1, 260, 1)), axis=2), 2)
    dup = inp.routes.copy()
    bad = inp.routes.copy()
    for i in range(260):
        row = dup[0, i]
        valid = row[(row >= 0) & (row < 300)]
        if len(valid):
            row[row == -1] = valid[-1]
    bad[bad == -1] = 300
    bad[0, ::2][bad[0, ::2] == 300] = -77
    for name, r in (("permuted", perm), ("duplicated", dup), ("invalid", bad)):
        other = DeviceRun(inp, 0.0625, routes=r, deterministic=True)
        for a, b in ((base.out, other.out), (base.out32, other.out32), (base.lse, other.lse),
                     (base.dq, other.dq), (base.dk, other.dk), (base.dv, other.dv)):
            assert torch.equal(a, b), name
        log(f"  {name}: bitwise identical")


def test_run_to_run_bitwise_determinism():
    # QSA_FLAG_DETERMINISTIC: every walk starts at the head of its key list.
    wl = synth.WORKLOADS[2]
    inp = synth.make_inputs(wl)
    a = DeviceRun(inp, wl.scale, deterministic=True)
    b = DeviceRun(inp, wl.scale, deterministic=True)
    for x, y in ((a.out32, b.out32), (a.lse, b.lse), (a.dq, b.dq), (a.dk, b.dk), (a.dv, b.dv)):
        assert torch.equal(x, y)


def test_default_walks_match_deterministic_walks():
    # The default mode takes the same sums in another order (rotated walks on
    # a workload with at least eight rows per resident wave): equal up to FP32
    # rounding, well inside the parity tolerances. The bound is the one the
    # parity tests use for the FP32 outputs (1e-3), taken 10 times tighter; a
    # chunk walked twice or skipped would miss it by orders of magnitude.
    wl = synth.WORKLOADS[3]
    inp = synth.make_inputs(wl)
    a = DeviceRun(inp, wl.scale, deterministic=True)
    b = DeviceRun(inp, wl.scale)
    assert not torch.equal(a.out32, b.out32)  # the walks were rotated
    for name, x, y in (("out_fp32", a.out32, b.out32), ("lse", a.lse, b.lse)):
        x = x.double()
        y = y.double()
        fin = torch.isfinite(x)
        assert torch.equal(fin, torch.isfinite(y)) and torch.equal(x[~fin], y[~fin]), name
        err = ((x - y)[fin].abs() / (1e-4 + 1e-4 * x[fin].abs())).max().item()
        log(f"  {name}: max |default - deterministic| / (1e-4 + 1e-4 |x|) = {err:.3f}")
        assert err <= 1.0, name
    for name, x, y in (("dq", a.dq, b.dq), ("dk", a.dk, b.dk), ("dv", a.dv, b.dv)):
        x = x.double()
        y = y.double()
        # bf16 outputs: one unit in the last place of either value, plus a
        # floor for values that are sums with cancellation (1e-3 of the
        # tensor's largest magnitude)
        bound = torch.maximum(x.abs(), y.abs()) * 2.0 ** -7 + 1e-3 * x.abs().max()
        assert ((x - y).abs() <= bound).all(), name


def test_nan_in_unselected_kv_does_not_leak():
    inp = synth.random_case(61, 1, 100, 120, 12, 1, 20)
    r = inp.routes.copy()
    r[(r >= 100) & (r < 120)] = -1                   # keys 100.. selected by nobody
    base = DeviceRun(inp, 0.0625, routes=r)
    k = inp.k.copy()
    v = inp.v.copy()
    k[0, 100:] = 0x7FC0                              # NaN
    v[0, 105:] = 0x7F80                              # +inf
    q = inp.q.copy()
    empty = np.nonzero(~((r >= 0) & (r < 120)).any(-1)[0])[0]
    q[0, empty] = 0x7FC0                             # Q of padding rows is irrelevant
    nan_inp = synth.Inputs(inp.wl, r, q, k, v, inp.grad_out, {})
    other = DeviceRun(nan_inp, 0.0625)
    for a, b in ((base.out32, other.out32), (base.lse, other.lse), (base.dq, other.dq),
                 (base.dv, other.dv)):
        assert torch.equal(a, b)
    assert torch.equal(base.dk[:, :100], other.dk[:, :100])
    assert (other.dk[:, 100:] == 0).all() and (other.dv[:, 100:] == 0).all()


def test_membership_offsets_beyond_int32():
    # B * Sq * stride > 2^31: the tail rows must still see their own routes.
    Sq = Skv = 46400
    W = 4
    rng = np.random.default_rng(3)
    routes = np.full((1, Sq, W), -1, np.int32)
    tail = np.arange(Sq - 300, Sq)
    routes[0, tail, 0] = tail
    routes[0, tail, 1] = rng.integers(0, Skv, size=len(tail))
    routes[0, tail, 2] = np.maximum(tail - 1, 0)
    log("membership beyond 2^31 bytes")
    P = qsa.preprocess(torch.from_numpy(routes).cuda(), Skv, with_row_keys=True)
    stride = P["memb"].shape[2]
    assert Sq * stride > 2**31
    memb_tail = P["memb"][0, Sq - 300:].cpu().numpy()
    rk = P["row_keys"][0, Sq - 300:].cpu().numpy()
    for n, i in enumerate(tail):
        want = oracle.route_set(routes, Skv, int(i))
        got = np.nonzero(memb_tail[n])[0]
        assert np.array_equal(got, want), int(i)
        assert np.array_equal(rk[n, :len(want)], want)
    del P
    torch.cuda.empty_cache()
    # forward on the same routes (small head count, D=256): tail rows vs oracle
    q = synth.bf16_bits(rng.standard_normal((1, Sq, 12, 256), dtype=np.float32))
    kv = synth.bf16_bits(rng.standard_normal((1, Skv, 1, 256), dtype=np.float32))
    inp = synth.Inputs(None, routes, q, kv, kv, None, {})
    run = DeviceRun(inp, 0.0625, backward=False)
    Pr = oracle.Problem(q, kv, kv, routes, 0.0625)
    rows = tail[-40:]
    o_ref, l_ref = Pr.forward(rows)
    check_close("out_fp32[tail]", to_np(run.out32[0, rows]), o_ref, TOL_FP32)


def test_errors_through_binding():
    q = torch.zeros((1, 8, 12, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((1, 8, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        qsa.forward(q, k, k, r, 0.1)
    q = torch.zeros((1, 8, 12, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, 1, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        qsa.forward(q, k, k, r, float("inf"))
    with pytest.raises(TypeError):
        qsa.forward(q, k, k, r.float(), 0.1)
    with pytest.raises(TypeError):
        qsa.forward(q.float(), k, k, r, 0.1)
