"""Helpers for the GPU parity tests: move seeded inputs to the GPU, run the HIP
path through the binding, and compare against the oracle with the stated
tolerances (|x - ref| <= tol + tol * |ref| elementwise; -inf matches -inf)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from token_indexed_sparse_amd import qsa, synth

TOL_BF16 = 2e-2
TOL_FP32 = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceRun:
    """Inputs on the GPU and the outputs of one forward + backward."""

    def __init__(self, inp: synth.Inputs, scale: float, routes: np.ndarray = None,
                 backward: bool = True, deterministic: bool = False):
        r = inp.routes if routes is None else routes
        self.q = to_gpu_bf16(inp.q)
        self.k = to_gpu_bf16(inp.k)
        self.v = to_gpu_bf16(inp.v)
        self.g = to_gpu_bf16(inp.grad_out) if inp.grad_out is not None else None
        self.routes = torch.from_numpy(np.ascontiguousarray(r)).cuda()
        self.scale = scale
        self.out, self.out32, self.lse = qsa.forward(self.q, self.k, self.v, self.routes, scale,
                                                     deterministic=deterministic)
        if backward and self.g is not None:
            self.dq, self.dk, self.dv = qsa.backward(self.g, self.q, self.k, self.v, self.out32,
                                                     self.lse, self.routes, scale,
                                                     deterministic=deterministic)
        torch.cuda.synchronize()


def check_close(name: str, x: np.ndarray, ref: np.ndarray, tol: float) -> dict:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (name, x.shape, ref.shape)
    same_inf = np.isinf(ref) & (x == ref)
    fin = np.isfinite(ref)
    # differences only where the reference is finite (-inf lse of empty rows
    # compares by equality above)
    diff = np.subtract(x, ref, out=np.zeros_like(ref), where=fin)
    err = np.where(fin, np.abs(diff), np.inf)
    ok = same_inf | (err <= tol + tol * np.abs(np.where(fin, ref, 0.0)))
    stats = {
        "max_abs": float(np.max(np.where(fin, err, 0.0))) if x.size else 0.0,
        "norm_rel": float(np.linalg.norm(diff) /
                          max(np.linalg.norm(np.where(fin, ref, 0)), 1e-300)) if x.size else 0.0,
    }
    if not ok.all():
        bad = np.argwhere(~ok)
        first = [tuple(int(v) for v in b) for b in bad[:5]]
        vals = [(float(x[b]), float(ref[b])) for b in map(tuple, bad[:5])]
        raise AssertionError(f"{name}: {len(bad)} of {x.size} outside tol {tol}: first {first} "
                             f"(got, ref) {vals}; stats {stats}")
    log(f"  {name}: ok max_abs={stats['max_abs']:.3e} norm_rel={stats['norm_rel']:.3e}")
    return stats


def check_preprocess_exact(routes_np: np.ndarray, Skv: int, routes_gpu: torch.Tensor) -> None:
    """Membership, tile kinds, tile lists and per-row key lists, bit-exact."""
    import oracle
    P = qsa.preprocess(routes_gpu, Skv)
    torch.cuda.synchronize()
    memb_ref, has_ref = oracle.membership(routes_np, Skv)
    memb = P["memb"].cpu().numpy()
    assert memb.shape == memb_ref.shape
    if not np.array_equal(memb, memb_ref):
        bad = np.argwhere(memb != memb_ref)
        raise AssertionError(f"membership differs at {len(bad)} cells, first {bad[:5].tolist()}")
    del memb
    assert np.array_equal(P["has_routes"].cpu().numpy(), has_ref)
    T = oracle.tiles(memb_ref, Skv)
    del memb_ref
    for name, ref in T.items():
        got = P[name].cpu().numpy()
        assert np.array_equal(got, ref), f"{name} differs"
    rk = P["row_keys"].cpu().numpy()
    rc = P["row_cnt"].cpu().numpy()
    B, Sq, W = routes_np.shape
    for row in range(B * Sq):
        want = oracle.route_set(routes_np, Skv, row)
        got = rk.reshape(-1, W)[row]
        n = len(want)
        assert rc.reshape(-1)[row] == n, f"row_cnt row {row}"
        assert np.array_equal(got[:n], want) and (got[n:] == -1).all(), f"row_keys row {row}"
    log(f"  preprocess bit-exact: memb {memb_ref_shape(routes_np, Skv)}, "
        f"kinds {T['kinds'].shape}, {B * Sq} row lists")


def memb_ref_shape(routes_np, Skv):
    B, Sq, _ = routes_np.shape
    return (B, Sq, -(-Skv // 128) * 128)
