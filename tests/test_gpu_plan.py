"""Route plans (qsa_plan_build and the planned calls) on an MI355X.

The plan's tables must equal the oracle's bit for bit (membership bits, tile
kinds, tile lists, per-row key lists). The planned calls must give bitwise the
results of the plain calls on the same routes in the deterministic mode, for a
forward, a recomputed forward and a backward on one plan, and a rebuilt plan
in the same buffer must serve other routes.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_FP32, DeviceRun, check_close, log, to_gpu_bf16, to_np
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _check_tables(routes_np: np.ndarray, Skv: int, plan: qsa.Plan) -> None:
    T = qsa.plan_tables(plan)
    torch.cuda.synchronize()
    memb_ref, _ = oracle.membership(routes_np, Skv)
    # bit (j % 32) of word j / 32: little-endian bit order within little-endian words
    bits_ref = np.packbits(memb_ref, axis=-1, bitorder="little").view("<u4")
    assert np.array_equal(T["mbits"].cpu().numpy().view(np.uint32), bits_ref), "mbits"
    tiles = oracle.tiles(memb_ref, Skv)
    for name, ref in tiles.items():
        assert np.array_equal(T[name].cpu().numpy(), ref), name
    rk = T["row_keys"].cpu().numpy()
    rc = T["row_cnt"].cpu().numpy().reshape(-1)
    B, Sq, W = routes_np.shape
    for row in range(B * Sq):
        want = oracle.route_set(routes_np, Skv, row)
        n = len(want)
        got = rk.reshape(-1, W)[row]
        assert rc[row] == n, f"row_cnt row {row}"
        assert np.array_equal(got[:n], want) and (got[n:] == -1).all(), f"row_keys row {row}"
    log(f"  plan tables bit-exact: {B * Sq} rows, kinds {tiles['kinds'].shape}")


CASES = [
    ("random", dict(seed=61, B=2, Sq=300, Skv=333, Hq=24, Hkv=2, W=40)),
    ("tiled", dict(seed=62, B=1, Sq=384, Skv=512, Hq=12, Hkv=1, p_full=0.5, extra=20)),
]


def _inputs(kind, case):
    return synth.random_case(**case) if kind == "random" else synth.tiled_case(**case)


@pytest.mark.parametrize("kind,case", CASES, ids=[c[0] for c in CASES])
def test_plan_tables_match_oracle(kind, case):
    log(f"plan tables {kind} {case}")
    inp = _inputs(kind, case)
    routes = torch.from_numpy(inp.routes).cuda()
    plan = qsa.plan_build(routes, case["Skv"], Hkv=case["Hkv"])
    _check_tables(inp.routes, case["Skv"], plan)


@pytest.mark.parametrize("kind,case", CASES, ids=[c[0] for c in CASES])
def test_planned_calls_match_plain_calls_bitwise(kind, case):
    log(f"planned calls {kind} {case}")
    inp = _inputs(kind, case)
    scale = 0.0625
    ref = DeviceRun(inp, scale, deterministic=True)
    plan = qsa.plan_build(ref.routes, case["Skv"], Hkv=case["Hkv"], deterministic=True)
    # forward, then the recompute a checkpointed layer runs, then the backward
    for _ in range(2):
        out, out32, lse = qsa.forward_planned(plan, ref.q, ref.k, ref.v, scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref.out) and torch.equal(out32, ref.out32)
        assert torch.equal(lse, ref.lse)
    dq, dk, dv = qsa.backward_planned(plan, ref.g, ref.q, ref.k, ref.v, out32, lse, scale)
    torch.cuda.synchronize()
    assert torch.equal(dq, ref.dq) and torch.equal(dk, ref.dk) and torch.equal(dv, ref.dv)
    log("  planned forward x2 and backward bitwise equal to the plain calls")


def test_plan_buffer_rebuilt_for_other_routes():
    """One plan buffer, two builds: the second (smaller) routes replace the first,
    and the planned calls match the oracle on them."""
    a = synth.random_case(63, 1, 400, 500, 12, 1, 60)
    b = synth.random_case(64, 1, 150, 260, 12, 1, 25)
    dims_a = qsa.make_dims(1, 400, 500, 12, 1, 256, 60)
    mem = torch.empty(qsa.plan_bytes(dims_a), dtype=torch.uint8, device="cuda")
    plan_a = qsa.plan_build(torch.from_numpy(a.routes).cuda(), 500, plan_mem=mem)
    assert plan_a.mem.data_ptr() == mem.data_ptr()
    qa = to_gpu_bf16(a.q)
    ka, va = to_gpu_bf16(a.k), to_gpu_bf16(a.v)
    out_a = qsa.forward_planned(plan_a, qa, ka, va, 0.0625)[1]
    torch.cuda.synchronize()
    plan_b = qsa.plan_build(torch.from_numpy(b.routes).cuda(), 260, plan_mem=mem)
    assert plan_b.mem.data_ptr() == mem.data_ptr()
    _check_tables(b.routes, 260, plan_b)
    q, k, v, g = (to_gpu_bf16(x) for x in (b.q, b.k, b.v, b.grad_out))
    out, out32, lse = qsa.forward_planned(plan_b, q, k, v, 0.0625)
    dq, dk, dv = qsa.backward_planned(plan_b, g, q, k, v, out32, lse, 0.0625)
    torch.cuda.synchronize()
    P = oracle.Problem(b.q, b.k, b.v, b.routes, 0.0625, b.grad_out)
    o_ref, l_ref = P.forward_full()
    check_close("out_fp32", to_np(out32), o_ref, TOL_FP32)
    check_close("lse", to_np(lse), l_ref, TOL_FP32)
    dq_ref, dk_ref, dv_ref = P.backward_full()
    check_close("dq", to_np(dq), dq_ref, TOL_BF16)
    check_close("dk", to_np(dk), dk_ref, TOL_BF16)
    check_close("dv", to_np(dv), dv_ref, TOL_BF16)
    # the first routes' result was computed before the rebuild
    Pa = oracle.Problem(a.q, a.k, a.v, a.routes, 0.0625)
    check_close("out_fp32 (first routes)", to_np(out_a), Pa.forward_full()[0], TOL_FP32)


def test_planned_calls_check_tensor_shapes_against_the_plan():
    inp = synth.random_case(65, 1, 100, 130, 12, 1, 20)
    plan = qsa.plan_build(torch.from_numpy(inp.routes).cuda(), 130)
    q, k, v = (to_gpu_bf16(x) for x in (inp.q, inp.k, inp.v))
    with pytest.raises(ValueError):
        qsa.forward_planned(plan, q[:, :50], k, v)
    with pytest.raises(ValueError):
        qsa.forward_planned(plan, q, k[:, :100], v[:, :100])
