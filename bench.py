"""Benchmark: QSA forward + backward on one MI355X.

One step = qsa_forward + qsa_backward on one batch of resident synthetic
inputs, each call with its own route preprocessing, delta and casts (the full
call, as the cuDNN Frontend QSA page's "Support and execution" section asks for
benchmarks). Outputs and workspaces are allocated before the timed region.

Prints one JSON line:
  value      sparse TFLOP/s = (4 + 10) * Hq * 256 * nnz / step time, with nnz the
             number of distinct valid (query, key) pairs of the routes
  roofline   the longest-running kernel: algorithmic FLOP per launch / its
             average duration measured with HIP events on its own stream,
             against the MI355X dense bf16 MFMA peak; `traffic` is its HBM
             bytes per launch from the committed rocprofv3 counter summary
             (profiles/traffic_<workload>.txt), null once the kernels changed
  cpu_baseline  the FP64 oracle on a bounded sample of the same workload,
             on this host's cores, scaled to TFLOP/s
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "QSA fwd+bwd sparse TFLOP/s (12Q/1KV, d=256) and % of MFMA peak, 1 GPU"

# Algorithmic FLOP per (distinct valid pair, query head), by kernel, and which
# pairs each kernel computes: "partial" = pairs outside full 128 x 128 tiles
# (gathered kernels), "full" = pairs inside them (dense kernels).
FLOP_PER_PAIR_HEAD = {
    "forward": 4 * 256,        # S = QK^T and O = PV
    "forward_dense": 4 * 256,
    "dq": 6 * 256,             # S, dP = dO V^T, dQ = dS K
    "dq_dense": 6 * 256,
    "dkdv": 8 * 256,           # S, dP, dV = P^T dO, dK = dS^T Q
    "dkdv_dense": 8 * 256,
}
KERNEL_PAIRS = {"forward": "partial", "forward_dense": "full", "dq": "partial",
                "dq_dense": "full", "dkdv": "partial", "dkdv_dense": "full"}
COUNTED_FWD = 4 * 256
COUNTED_BWD = 10 * 256
FWD_STAGES = ["preprocess_fwd", "forward", "forward_dense"]
BWD_STAGES = ["preprocess_bwd", "delta", "dq", "dq_dense", "dkdv", "dkdv_dense", "dkdv_reduce"]


def pairs_per_row(routes: np.ndarray, Skv: int) -> np.ndarray:
    """Distinct valid keys per query row; their sum is the sparse work of a step."""
    r = routes.reshape(-1, routes.shape[-1])
    out = np.empty(r.shape[0], np.int64)
    for a in range(0, r.shape[0], 4096):
        c = r[a:a + 4096].astype(np.int64)
        s = np.sort(np.where((c >= 0) & (c < Skv), c, -1), axis=-1)
        out[a:a + 4096] = (s[:, 0] >= 0) + ((s[:, 1:] != s[:, :-1]) & (s[:, 1:] >= 0)).sum(1)
    return out


def full_tile_pairs(routes: np.ndarray, Sq: int, Skv: int) -> int:
    """Pairs inside full 128 x 128 tiles (every row of the query tile selects every key of
    the key tile; edge tiles are never full)."""
    B = routes.shape[0]
    nQT, nKT = (Sq + 127) // 128, (Skv + 127) // 128
    total = 0
    for b in range(B):
        cnt = np.zeros((nQT, nKT), np.int64)
        r = routes[b]
        for a in range(0, Sq, 1024):
            c = r[a:a + 1024].astype(np.int64)
            s = np.sort(np.where((c >= 0) & (c < Skv), c, -1), axis=-1)
            keep = s >= 0
            keep[:, 1:] &= s[:, 1:] != s[:, :-1]
            rows = np.broadcast_to(np.arange(a, a + c.shape[0])[:, None] // 128, s.shape)
            np.add.at(cnt, (rows[keep], s[keep] // 128), 1)
        total += int((cnt == 128 * 128).sum()) * 128 * 128
    return total


TRAFFIC_SOURCES = ("token_indexed_sparse_amd/csrc/common.h", "token_indexed_sparse_amd/csrc/bwd.hip",
                   "token_indexed_sparse_amd/csrc/fwd.hip", "token_indexed_sparse_amd/csrc/dense.hip")


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE) from the
    committed rocprofv3 summary, or None if there is none or the kernels changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    sha, rows = None, {}
    for line in open(path):
        parts = line.split()
        if line.startswith("source_sha256:"):
            sha = parts[1]
        elif line.startswith("traffic ") and len(parts) == 4:
            rows[parts[1]] = int(parts[2]) + int(parts[3])
    if sha != h.hexdigest():
        return None
    return rows.get("k_" + kernel)


def hip_runtime():
    lib = None
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            lib = ctypes.CDLL(line.split()[-1])
            break
    if lib is None:
        lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.restype = ctypes.c_int
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.restype = ctypes.c_int
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    return lib


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h.value

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]),
                                            ctypes.c_void_p(self.ev[b])) == 0
        return ms.value


def cpu_baseline(inp, wl, nnz_row: np.ndarray, seconds: float) -> dict:
    """The oracle (fwd + full bwd of a sample of query rows), timed on host cores."""
    import oracle
    P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, wl.scale, inp.grad_out)
    rng = np.random.default_rng(0)
    rows_all = np.nonzero(nnz_row > 0)[0]
    # calibrate on a few rows, then size the sample to the time budget
    probe = rng.choice(rows_all, min(4, len(rows_all)), replace=False)
    t = time.perf_counter()
    P.backward_rows(probe)
    per_row = (time.perf_counter() - t) / len(probe)
    n = int(max(4, min(len(rows_all), seconds / max(per_row, 1e-9))))
    rows = np.sort(rng.choice(rows_all, n, replace=False))
    t = time.perf_counter()
    P.backward_rows(rows)
    dt = time.perf_counter() - t
    flop = (COUNTED_FWD + COUNTED_BWD) * wl.Hq * float(nnz_row[rows].sum())
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"forward + full backward (dq and the rows' dk/dv contributions) of {n} "
                      f"random query rows of {wl.name} ({int(nnz_row[rows].sum())} pairs), "
                      f"FP64 C oracle, one thread, {dt:.1f} s",
            "host_threads_available": os.cpu_count()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_t32768_12q1kv",
                    help="workload name or index 1-5 (default: the 32k-token long-context one)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--deterministic", action="store_true",
                    help="set QSA_FLAG_DETERMINISTIC (head-first key walks, bitwise reproducible)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n}), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU sharding in this build)", file=sys.stderr)
        return 2

    import torch
    from token_indexed_sparse_amd import qsa, synth

    wl = None
    for idx, w in synth.WORKLOADS.items():
        if args.workload in (w.name, str(idx)):
            wl = w
    if wl is None:
        raise SystemExit(f"unknown workload {args.workload}")
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl)
    nnz_row = pairs_per_row(inp.routes, wl.Skv)
    nnz = int(nnz_row.sum())
    nnz_full = full_tile_pairs(inp.routes, wl.Sq, wl.Skv)
    pairs = {"all": nnz, "full": nnz_full, "partial": nnz - nnz_full}

    dev = torch.device("cuda:0")

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, g = bf(inp.q), bf(inp.k), bf(inp.v), bf(inp.grad_out)
    routes = torch.from_numpy(inp.routes).to(dev)
    out = torch.empty_like(q)
    out32 = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty((wl.B, wl.Hq, wl.Sq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dims = qsa.make_dims(wl.B, wl.Sq, wl.Skv, wl.Hq, wl.Hkv, wl.D, wl.W,
                         deterministic=args.deterministic)
    ws_f = torch.empty(qsa.forward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(qsa.backward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    lib = qsa.library()
    lib.qsa_forward_timed.restype = ctypes.c_int
    lib.qsa_forward_timed.argtypes = [ctypes.POINTER(qsa.Dims)] + [ctypes.c_void_p] * 4 + [
        ctypes.c_float] + [ctypes.c_void_p] * 3 + [ctypes.c_void_p, ctypes.c_size_t,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_int32]
    lib.qsa_backward_timed.restype = ctypes.c_int
    lib.qsa_backward_timed.argtypes = [ctypes.POINTER(qsa.Dims)] + [ctypes.c_void_p] * 7 + [
        ctypes.c_float] + [ctypes.c_void_p] * 3 + [ctypes.c_void_p, ctypes.c_size_t,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_int32]
    hip = hip_runtime()
    stream = torch.cuda.current_stream().cuda_stream
    K, W = args.steps, args.warmup
    NF, NB = len(FWD_STAGES), len(BWD_STAGES)
    fev = [Events(hip, NF + 1) for _ in range(K)]
    bev = [Events(hip, NB + 1) for _ in range(K)]

    def step(i=None):
        fe = ctypes.cast(fev[i].ev, ctypes.c_void_p) if i is not None else None
        be = ctypes.cast(bev[i].ev, ctypes.c_void_p) if i is not None else None
        st = lib.qsa_forward_timed(ctypes.byref(dims), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   routes.data_ptr(), wl.scale, out.data_ptr(), out32.data_ptr(),
                                   lse.data_ptr(), ws_f.data_ptr(), ws_f.numel(), stream,
                                   fe, NF + 1 if fe is not None else 0)
        assert st == 0, st
        st = lib.qsa_backward_timed(ctypes.byref(dims), g.data_ptr(), q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), out32.data_ptr(), lse.data_ptr(),
                                    routes.data_ptr(), wl.scale, dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), ws_b.data_ptr(), ws_b.numel(), stream,
                                    be, NB + 1 if be is not None else 0)
        assert st == 0, st

    print(f"[bench] warmup {W}", file=sys.stderr, flush=True)
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    stage_ms = {}
    for a, name in enumerate(FWD_STAGES):
        stage_ms[name] = float(np.mean([e.elapsed(a, a + 1) for e in fev]))
    for a, name in enumerate(BWD_STAGES):
        stage_ms[name] = float(np.mean([e.elapsed(a, a + 1) for e in bev]))
    fwd_ms = float(np.mean([e.elapsed(0, NF) for e in fev]))
    bwd_ms = float(np.mean([e.elapsed(0, NB) for e in bev]))
    flop_fwd = COUNTED_FWD * wl.Hq * nnz
    flop_bwd = COUNTED_BWD * wl.Hq * nnz
    value = (flop_fwd + flop_bwd) / (ms_step * 1e-3) / 1e12

    dom = max(KERNEL_PAIRS, key=lambda s: stage_ms[s])
    dom_flop = FLOP_PER_PAIR_HEAD[dom] * wl.Hq * pairs[KERNEL_PAIRS[dom]]
    achieved = dom_flop / (stage_ms[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(wl.name, dom),
                "flop_per_launch": dom_flop, "avg_launch_ms": stage_ms[dom]}

    # algorithmic HBM bytes of one step (each tensor once per call, membership once per call)
    Bq = wl.B * wl.Sq * wl.Hq * wl.D
    Bk = wl.B * wl.Skv * wl.Hkv * wl.D
    memb = wl.B * wl.Sq * (-(-wl.Skv // 128) * 128)
    rt = inp.routes.nbytes
    fwd_bytes = rt + memb + 2 * Bq + 2 * 2 * Bk + 2 * Bq + 4 * Bq + 4 * wl.B * wl.Hq * wl.Sq
    bwd_bytes = (rt + memb + 2 * Bq + 2 * 2 * Bk + 2 * Bq + 4 * Bq + 4 * wl.B * wl.Hq * wl.Sq
                 + 2 * 4 * wl.B * wl.Hq * wl.Sq + 2 * Bq + 2 * 2 * Bk)

    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Sq": wl.Sq, "Skv": wl.Skv, "Hq": wl.Hq,
                   "Hkv": wl.Hkv, "D": wl.D, "W": wl.W, "nnz_pairs": nnz, "full_tile_pairs": nnz_full,
                   "flop_per_step": flop_fwd + flop_bwd, "parallelism": "single GPU",
                   "deterministic": bool(args.deterministic)},
        "mfma_peak_frac": value / PEAK_BF16_TFLOPS,
        "forward_tflops": flop_fwd / (fwd_ms * 1e-3) / 1e12,
        "backward_tflops": flop_bwd / (bwd_ms * 1e-3) / 1e12,
        "stage_ms": stage_ms,
        "algorithmic_hbm_gbs": (fwd_bytes + bwd_bytes) / (ms_step * 1e-3) / 1e9,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, wl, nnz_row, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
