"""Block-bitmap entry points (qsa_block_plan_build, qsa_block_forward,
qsa_block_backward) on an MI355X.

* A hand-built selection (bounds, out-of-range block numbers, floor rounding,
  a sequence whose first token is not a multiple of four) and a packed
  document workload: outputs against the oracle's Miles lookup, to the usual
  tolerances, and the block plan's tables bit for bit.
* The seeded workloads 1-4 re-expressed as packed sequences with a bitmap
  built from the drawn block numbers: the block calls must give bitwise the
  results of the route calls on the same selection written as packed route
  rows (deterministic mode), which the route parity tests tie to the oracle.
  Workload 5 (a query shard of 4096 rows against 32768 keys) has no packed
  form: the block interface takes the same T tokens as queries and keys.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_FP32, check_close, log, to_gpu_bf16, to_np
from test_block_pins import HAND_NB, HAND_T, _hand
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _meta_gpu(sel, lo, hi, bb, tb, bf, bl):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (sel, lo, hi, bb, tb, bf, bl)]


def _check_block_tables(plan, memb_ref, T):
    Tb = qsa.plan_tables(plan)
    torch.cuda.synchronize()
    bits_ref = np.packbits(memb_ref, axis=-1, bitorder="little").view("<u4")
    assert np.array_equal(Tb["mbits"].cpu().numpy().view(np.uint32), bits_ref), "mbits"
    for name, ref in oracle.tiles(memb_ref, T).items():
        assert np.array_equal(Tb[name].cpu().numpy(), ref), name
    rk = Tb["row_keys"].cpu().numpy()[0]
    rc = Tb["row_cnt"].cpu().numpy()[0]
    m = memb_ref[0, :, :T] != 0
    for t in range(T):
        want = np.nonzero(m[t])[0]
        assert rc[t] == len(want), f"row_cnt {t}"
        assert np.array_equal(rk[t, :len(want)], want) and (rk[t, len(want):] == -1).all(), t
    log(f"  block plan tables bit-exact: T={T}")


def _oracle_compare(q, k, v, g, memb, scale, got):
    routes = oracle.routes_from_membership(memb, memb.shape[1])
    P = oracle.Problem(q[None], k[None], v[None], routes, scale, g[None])
    o_ref, l_ref = P.forward_full()
    out, out32, lse, dq, dk, dv = got
    check_close("out_fp32", to_np(out32)[None], o_ref, TOL_FP32)
    check_close("lse", to_np(lse)[None], l_ref, TOL_FP32)
    check_close("out", to_np(out)[None], o_ref, TOL_BF16)
    dq_ref, dk_ref, dv_ref = P.backward_full()
    check_close("dq", to_np(dq)[None], dq_ref, TOL_BF16)
    check_close("dk", to_np(dk)[None], dk_ref, TOL_BF16)
    check_close("dv", to_np(dv)[None], dv_ref, TOL_BF16)


def _run_block(q, k, v, g, meta, scale, deterministic=False):
    out, out32, lse = qsa.block_forward(q, k, v, *meta, scale, deterministic=deterministic)
    dq, dk, dv = qsa.block_backward(g, q, k, v, out32, lse, *meta, scale,
                                    deterministic=deterministic)
    torch.cuda.synchronize()
    return out, out32, lse, dq, dk, dv


def test_hand_selection_against_oracle():
    sel, (lo, hi, bb, tb) = _hand()
    bf = np.array([0, 4, 6], np.int32)
    bl = np.array([3, 5, 9], np.int32)
    rng = np.random.default_rng(71)
    x = [synth.bf16_bits(rng.standard_normal(s, dtype=np.float32))
         for s in ((HAND_T, 12, 256), (HAND_T, 1, 256), (HAND_T, 1, 256), (HAND_T, 12, 256))]
    q, k, v, g = (to_gpu_bf16(a) for a in x)
    meta = _meta_gpu(sel, lo, hi, bb, tb, bf, bl)
    got = _run_block(q, k, v, g, meta, 0.0625)
    memb, _ = oracle.block_membership(sel, lo, hi, bb, tb)
    _oracle_compare(*x, memb, 0.0625, got)
    # rows without an allowed key: zero output, -inf lse, zero dq
    for t in (1, 6, 9):
        assert torch.count_nonzero(got[1][t]) == 0 and torch.isneginf(got[2][:, t]).all()
        assert torch.count_nonzero(got[3][t]) == 0
    plan = qsa.block_plan_build(*meta)
    _check_block_tables(plan, memb, HAND_T)
    assert plan.dims.W == min(HAND_T, 4 * HAND_NB)


def test_packed_documents_against_oracle():
    wl = synth.Workload("docs_300", 1, 300, 300, 12, 1, 256, 8, "docs", 7, n_docs=5)
    bi = synth.block_inputs(synth.make_inputs(wl, record_blocks=True))
    meta = _meta_gpu(bi.sel_blocks, bi.lo, bi.hi, bi.blk_base, bi.tok_base, bi.block_first,
                     bi.block_last)
    q, k, v, g = (to_gpu_bf16(a[0]) for a in (bi.q, bi.k, bi.v, bi.grad_out))
    got = _run_block(q, k, v, g, meta, wl.scale)
    memb, _ = oracle.block_membership(bi.sel_blocks, bi.lo, bi.hi, bi.blk_base, bi.tok_base)
    _oracle_compare(bi.q[0], bi.k[0], bi.v[0], bi.grad_out[0], memb, wl.scale, got)
    _check_block_tables(qsa.block_plan_build(*meta), memb, bi.T)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_workloads_as_bitmaps_match_route_calls_bitwise(idx):
    wl = synth.WORKLOADS[idx]
    log(f"workload {wl.name} as a block bitmap")
    bi = synth.block_inputs(synth.make_inputs(wl, record_blocks=True))
    log(f"  T={bi.T} NB={bi.NB}")
    meta = _meta_gpu(bi.sel_blocks, bi.lo, bi.hi, bi.blk_base, bi.tok_base, bi.block_first,
                     bi.block_last)
    q, k, v, g = (to_gpu_bf16(a[0]) for a in (bi.q, bi.k, bi.v, bi.grad_out))
    blk = _run_block(q, k, v, g, meta, wl.scale, deterministic=True)
    routes = torch.from_numpy(bi.routes).cuda()
    out, out32, lse = qsa.forward(q[None], k[None], v[None], routes, wl.scale, deterministic=True)
    dq, dk, dv = qsa.backward(g[None], q[None], k[None], v[None], out32, lse, routes, wl.scale,
                              deterministic=True)
    torch.cuda.synchronize()
    for name, a, b in (("out", blk[0], out[0]), ("out_fp32", blk[1], out32[0]),
                       ("lse", blk[2], lse[0]), ("dq", blk[3], dq[0]), ("dk", blk[4], dk[0]),
                       ("dv", blk[5], dv[0])):
        assert torch.equal(a, b), name
    log("  block and route calls bitwise equal")
    if bi.T <= 16384:
        memb, _ = oracle.block_membership(bi.sel_blocks, bi.lo, bi.hi, bi.blk_base, bi.tok_base)
        _check_block_tables(qsa.block_plan_build(*meta), memb, bi.T)


@pytest.mark.parametrize("seed,T,NB", [(81, 300, 90), (82, 700, 40), (83, 129, 200)])
def test_random_metadata_against_oracle(seed, T, NB):
    """Arbitrary metadata (the page leaves it a caller contract): lo > hi, bounds past
    the tokens, block bases below 0 and past NB, token origins off the four-token
    grid. The block calls must select exactly what the oracle's lookup selects."""
    rng = np.random.default_rng(seed)
    sel = (rng.random((T, NB)) < 0.3).astype(np.uint8) * rng.integers(1, 256, (T, NB),
                                                                      dtype=np.uint8)
    lo = rng.integers(-20, T + 20, T).astype(np.int32)
    hi = rng.integers(-20, T + 20, T).astype(np.int32)
    bb = rng.integers(-10, NB + 10, T).astype(np.int32)
    tb = rng.integers(-30, T + 30, T).astype(np.int32)
    bf = np.arange(NB, dtype=np.int32) * 4
    bl = bf + 3
    x = [synth.bf16_bits(rng.standard_normal(s, dtype=np.float32))
         for s in ((T, 12, 256), (T, 1, 256), (T, 1, 256), (T, 12, 256))]
    q, k, v, g = (to_gpu_bf16(a) for a in x)
    meta = _meta_gpu(sel, lo, hi, bb, tb, bf, bl)
    got = _run_block(q, k, v, g, meta, 0.0625)
    memb, _ = oracle.block_membership(sel, lo, hi, bb, tb)
    _check_block_tables(qsa.block_plan_build(*meta), memb, T)
    _oracle_compare(*x, memb, 0.0625, got)
