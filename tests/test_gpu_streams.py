"""The backward's two streams (dQ passes on a second stream of the library,
forked after delta and joined before the reduce), on an MI355X.

* Calls from two host threads at once, each on its own torch stream, with
  different problems: each call's results must equal, bit for bit, those of the
  same call made alone (deterministic mode), so no call may pick up another
  call's fork or join.
* Work enqueued on the caller's stream after the backward must see its
  outputs: a copy made right after the call, on the same stream, equals the
  outputs read after a device-wide synchronisation.
* A backward on the null stream.
"""
import ctypes
import threading

import pytest
import torch

from gpu_util import log, to_gpu_bf16
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qsa.library()  # fails loudly if the HIP library is missing


def _problem(seed, Sq, Skv, W):
    c = synth.random_case(seed, 1, Sq, Skv, 12, 1, W)
    q, k, v, g = (to_gpu_bf16(x) for x in (c.q, c.k, c.v, c.grad_out))
    routes = torch.from_numpy(c.routes).cuda()
    return q, k, v, g, routes


def _step(prob, scale=0.0625):
    q, k, v, g, routes = prob
    out, o32, lse = qsa.forward(q, k, v, routes, scale, deterministic=True)
    dq, dk, dv = qsa.backward(g, q, k, v, o32, lse, routes, scale, deterministic=True)
    return dq, dk, dv


def test_two_threads_two_streams_match_calls_alone():
    probs = [_problem(201, 1500, 1500, 80), _problem(202, 2200, 1800, 120)]
    alone = []
    for p in probs:
        r = _step(p)
        torch.cuda.synchronize()
        alone.append([t.clone() for t in r])
    results = [[None] * 6 for _ in probs]
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(6):
                    r = _step(probs[i])
                    s.synchronize()
                    results[i][it] = [t.clone() for t in r]
        except Exception as e:  # reported below, from the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for i in range(2):
        for it in range(6):
            for name, a, b in zip(("dq", "dk", "dv"), results[i][it], alone[i]):
                assert torch.equal(a, b), (i, it, name)
    log("  two threads, two streams: every call equals the call alone")


def test_later_work_on_the_stream_sees_the_outputs():
    prob = _problem(203, 3000, 3000, 100)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dq, dk, dv = _step(prob)
        early = [t.clone() for t in (dq, dk, dv)]   # enqueued on s right after the call
    torch.cuda.synchronize()
    for a, b in zip(early, (dq, dk, dv)):
        assert torch.equal(a, b)


def test_backward_on_the_null_stream():
    prob = _problem(204, 1000, 1200, 60)
    ref = [t.clone() for t in _step(prob)]
    torch.cuda.synchronize()
    q, k, v, g, routes = prob
    out, o32, lse = qsa.forward(q, k, v, routes, 0.0625, deterministic=True)
    torch.cuda.synchronize()
    lib = qsa.library()
    dims = qsa.make_dims(1, q.shape[1], k.shape[1], 12, 1, 256, routes.shape[2],
                         deterministic=True)
    ws = torch.empty(qsa.backward_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = lib.qsa_backward(ctypes.byref(dims), g.data_ptr(), q.data_ptr(), k.data_ptr(),
                          v.data_ptr(), o32.data_ptr(), lse.data_ptr(), routes.data_ptr(), 0.0625,
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                          ws.numel(), None)
    assert st == 0, st
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)
