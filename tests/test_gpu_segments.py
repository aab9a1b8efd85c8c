"""Grouped dK/dV segments on an MI355X.

The gathered dK/dV pass takes its query rows in 2-tile segments grouped eight
tiles at a time; a group whose partial-tile rows select one of a 16-key group
more than 256 times runs each segment as its own work item, a lighter group runs
as one item. The case below is built so that both kinds occur (checked on the
CPU from the routes alone), and every output is compared with the oracle, in
the default and the deterministic mode; deterministic calls repeat bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_FP32, DeviceRun, check_close, log, to_np
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu

SPLIT_HITS = 256  # rows per (segment group, 16-key group) above which the group splits
GROUP_TILES = 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _split_groups(routes: np.ndarray, Skv: int) -> np.ndarray:
    """[query-tile group, 16-key group]: True where the rows of the group's
    partial tiles select a key of the 16-key group more than SPLIT_HITS times."""
    Sq = routes.shape[1]
    m = np.zeros((Sq, Skv), bool)
    for i in range(Sq):
        r = routes[0, i]
        r = r[(r >= 0) & (r < Skv)]
        m[i, r] = True
    nqt, nkt = -(-Sq // 128), -(-Skv // 128)
    kind = np.zeros((nqt, nkt), np.int8)  # 0 absent, 1 partial, 2 full
    for a in range(nqt):
        for b in range(nkt):
            blk = m[128 * a:128 * (a + 1), 128 * b:128 * (b + 1)]
            full = blk.shape == (128, 128) and blk.all()
            kind[a, b] = 2 if full else (1 if blk.any() else 0)
    ng = -(-nqt // GROUP_TILES)
    out = np.zeros((ng, -(-Skv // 16)), bool)
    for gq in range(ng):
        for kg in range(out.shape[1]):
            kt = (16 * kg) // 128
            hits = 0
            for qt in range(GROUP_TILES * gq, min(GROUP_TILES * (gq + 1), nqt)):
                if kind[qt, kt] == 1:
                    hits += int(m[128 * qt:128 * (qt + 1), 16 * kg:16 * (kg + 1)].any(1).sum())
            out[gq, kg] = hits > SPLIT_HITS
    return out


def test_split_and_merged_groups_match_the_oracle():
    # causal rows with 64 chosen blocks each: the first key groups are hit by
    # most later rows (split groups), the ones near the diagonal by few
    wl = synth.Workload("segments_s2048_12q1kv", 1, 2048, 2048, 12, 1, 256, 64, "single", 71)
    inp = synth.make_inputs(wl)
    split = _split_groups(inp.routes, wl.Skv)
    log(f"  split groups {int(split.sum())} of {split.size}")
    assert split.any() and (~split).any()
    P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, wl.scale, inp.grad_out)
    o_ref, l_ref, dq_ref, dk_ref, dv_ref = P.all_outputs()
    for det in (False, True):
        run = DeviceRun(inp, wl.scale, deterministic=det)
        tag = "deterministic " if det else ""
        check_close(f"{tag}out_fp32", to_np(run.out32), o_ref, TOL_FP32)
        check_close(f"{tag}lse", to_np(run.lse), l_ref, TOL_FP32)
        check_close(f"{tag}dq", to_np(run.dq), dq_ref, TOL_BF16)
        check_close(f"{tag}dk", to_np(run.dk), dk_ref, TOL_BF16)
        check_close(f"{tag}dv", to_np(run.dv), dv_ref, TOL_BF16)
        if det:
            again = DeviceRun(inp, wl.scale, deterministic=True)
            for a, b in ((run.dk, again.dk), (run.dv, again.dv), (run.dq, again.dq)):
                assert torch.equal(a, b)
