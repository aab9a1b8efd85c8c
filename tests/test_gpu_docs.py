"""Document-causal entry points (qsa_doc_plan_build, qsa_doc_forward,
qsa_doc_backward) on an MI355X.

* Small cases with padding tokens, documents of any layout and a query shard
  against all keys: outputs against the oracle's document-causal membership
  (to the usual tolerances) and the plan's tables bit for bit.
* Packed documents at 8192 tokens, and a 4096-query shard of a 32768-token
  sequence of documents: the document calls must give bitwise the results of
  the route calls on route rows that list each query's keys from its
  document's start (deterministic mode), which the route parity tests tie to
  the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_FP32, check_close, log, to_gpu_bf16, to_np
from test_doc_pins import _causal_routes, _doc_ids
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _tensors(rng, B, Sq, Skv, Hkv):
    x = [synth.bf16_bits(rng.standard_normal(s, dtype=np.float32))
         for s in ((B, Sq, 12 * Hkv, 256), (B, Skv, Hkv, 256), (B, Skv, Hkv, 256),
                   (B, Sq, 12 * Hkv, 256))]
    return x, [to_gpu_bf16(a) for a in x]


def _run_doc(q, k, v, g, qd, kd, start, scale, deterministic=False):
    out, out32, lse = qsa.doc_forward(q, k, v, qd, kd, scale, q_global_start=start,
                                      deterministic=deterministic)
    dq, dk, dv = qsa.doc_backward(g, q, k, v, out32, lse, qd, kd, scale, q_global_start=start,
                                  deterministic=deterministic)
    torch.cuda.synchronize()
    return out, out32, lse, dq, dk, dv


def _check_tables(plan, memb_ref, Skv):
    T = qsa.plan_tables(plan)
    torch.cuda.synchronize()
    bits_ref = np.packbits(memb_ref, axis=-1, bitorder="little").view("<u4")
    assert np.array_equal(T["mbits"].cpu().numpy().view(np.uint32), bits_ref), "mbits"
    for name, ref in oracle.tiles(memb_ref, Skv).items():
        assert np.array_equal(T[name].cpu().numpy(), ref), name
    rk = T["row_keys"].cpu().numpy()
    rc = T["row_cnt"].cpu().numpy()
    m = memb_ref[:, :, :Skv] != 0
    B, Sq = m.shape[:2]
    for b in range(B):
        for i in range(Sq):
            want = np.nonzero(m[b, i])[0]
            assert rc[b, i] == len(want)
            assert np.array_equal(rk[b, i, :len(want)], want) and (rk[b, i, len(want):] == -1).all()


CASES = [
    # padding and documents of any layout, self-attention
    dict(seed=91, B=2, Sq=300, Skv=300, Hkv=1, start=0, kind="random"),
    # a query shard (positions 500..699) against 700 keys, 24Q/2KV
    dict(seed=92, B=1, Sq=200, Skv=700, Hkv=2, start=500, kind="random"),
    # packed contiguous documents with a long one: full 128 x 128 tiles occur
    dict(seed=93, B=1, Sq=640, Skv=640, Hkv=1, start=0, kind="runs"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c['seed']}")
def test_small_cases_against_oracle(case):
    log(f"case {case}")
    rng = np.random.default_rng(case["seed"])
    B, Sq, Skv, start = case["B"], case["Sq"], case["Skv"], case["start"]
    if case["kind"] == "random":
        kd = rng.integers(0, 4, (B, Skv)).astype(np.int32)
    else:
        kd = np.stack([_doc_ids(np.array([0, 37, 420, 590]), Skv) for _ in range(B)])
        kd[:, 600:] = 0  # a padding tail
    qd = kd[:, start:start + Sq].copy()
    x, (q, k, v, g) = _tensors(rng, B, Sq, Skv, case["Hkv"])
    qd_t, kd_t = torch.from_numpy(qd).cuda(), torch.from_numpy(kd).cuda()
    got = _run_doc(q, k, v, g, qd_t, kd_t, start, 0.0625)
    memb, _ = oracle.doc_membership(qd, kd, start)
    if case["kind"] == "runs":
        tiles = oracle.tiles(memb, Skv)
        assert (tiles["kinds"] == 2).any(), "the case must have full tiles"
    routes = oracle.routes_from_membership(memb, Skv)
    P = oracle.Problem(*x[:3], routes, 0.0625, x[3])
    o_ref, l_ref = P.forward_full()
    check_close("out_fp32", to_np(got[1]), o_ref, TOL_FP32)
    check_close("lse", to_np(got[2]), l_ref, TOL_FP32)
    check_close("out", to_np(got[0]), o_ref, TOL_BF16)
    dq_ref, dk_ref, dv_ref = P.backward_full()
    check_close("dq", to_np(got[3]), dq_ref, TOL_BF16)
    check_close("dk", to_np(got[4]), dk_ref, TOL_BF16)
    check_close("dv", to_np(got[5]), dv_ref, TOL_BF16)
    # padding queries: zero output and gradient, -inf lse
    pad = torch.from_numpy(qd == 0).cuda()
    assert torch.count_nonzero(got[1][pad]) == 0 and torch.count_nonzero(got[3][pad]) == 0
    assert torch.isneginf(got[2].transpose(1, 2)[pad]).all()
    _check_tables(qsa.doc_plan_build(qd_t, kd_t, Hkv=case["Hkv"], q_global_start=start), memb,
                  Skv)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,Sq,n_docs,seed", [(8192, 8192, 4, 2), (32768, 4096, 8, 94)])
def test_documents_match_route_calls_bitwise(T, Sq, n_docs, seed):
    log(f"documents T={T} queries={Sq}")
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, T), n_docs - 1, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int64)
    ids = _doc_ids(starts, T)[None]
    start = T - Sq
    qd = ids[:, start:].copy()
    x, (q, k, v, g) = _tensors(rng, 1, Sq, T, 1)
    qd_t, kd_t = torch.from_numpy(qd).cuda(), torch.from_numpy(ids).cuda()
    got = _run_doc(q, k, v, g, qd_t, kd_t, start, 0.0625, deterministic=True)
    routes = torch.from_numpy(_causal_routes(starts, np.arange(start, T), T)).cuda()
    out, out32, lse = qsa.forward(q, k, v, routes, 0.0625, deterministic=True)
    dq, dk, dv = qsa.backward(g, q, k, v, out32, lse, routes, 0.0625, deterministic=True)
    torch.cuda.synchronize()
    for name, a, b in (("out", got[0], out), ("out_fp32", got[1], out32), ("lse", got[2], lse),
                       ("dq", got[3], dq), ("dk", got[4], dk), ("dv", got[5], dv)):
        assert torch.equal(a, b), name
    log("  document and route calls bitwise equal")
