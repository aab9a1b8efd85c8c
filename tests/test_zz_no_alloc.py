"""The allocation-free forward (qsa_forward_noalloc, fixed device scratch)
against the ordinary forward (caller workspace), through the C ABI.

Two calls in a row, the second smaller than the first, so the second runs on
scratch that still holds the first call's data. With QSA_FLAG_DETERMINISTIC
both entry points run the same kernels on the same inputs: the outputs must be
bitwise equal, and both must match the FP64 oracle within the parity
tolerances.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_FP32, check_close, log, to_gpu_bf16, to_np
from token_indexed_sparse_amd import qsa, synth

pytestmark = pytest.mark.gpu


def _run(case):
    inp = synth.random_case(**case)
    q, k, v = to_gpu_bf16(inp.q), to_gpu_bf16(inp.k), to_gpu_bf16(inp.v)
    routes = torch.from_numpy(inp.routes).cuda()
    ref = qsa.forward(q, k, v, routes, 0.0625, deterministic=True)
    out = torch.full_like(q, float("nan"))
    out32 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), dtype=torch.float32,
                     device="cuda")
    qsa.forward_noalloc(q, k, v, routes, 0.0625, out=out, out_fp32=out32, lse=lse,
                        deterministic=True)
    torch.cuda.synchronize()
    return inp, ref, (out, out32, lse)


def test_noalloc_forward_matches_forward_twice_second_smaller():
    torch.cuda.init()
    cases = [dict(seed=81, B=2, Sq=700, Skv=900, Hq=24, Hkv=2, W=120),
             dict(seed=82, B=1, Sq=150, Skv=333, Hq=12, Hkv=1, W=40)]
    for case in cases:
        log(f"noalloc case {case}")
        inp, ref, got = _run(case)
        for name, a, b in zip(("out", "out_fp32", "lse"), ref, got):
            assert torch.equal(a, b), name
        P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, 0.0625)
        o_ref, l_ref = P.forward_full()
        check_close("out_fp32", to_np(got[1]), o_ref, TOL_FP32)
        check_close("lse", to_np(got[2]), l_ref, TOL_FP32)
        check_close("out", to_np(got[0]), o_ref, TOL_BF16)


def test_noalloc_rejects_calls_beyond_the_scratch():
    q = torch.zeros((1, 32768, 12, 256), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 32768, 1, 256), dtype=torch.bfloat16, device="cuda")
    r = torch.full((1, 32768, 2052), -1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 12, 32768), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        qsa.forward_noalloc(q, kv, kv, r, 0.0625, out=out, out_fp32=out32, lse=lse)
