"""Benchmark: QSA forward + backward on one MI355X.

One step = qsa_plan_build + qsa_forward_planned + qsa_backward_planned on one
batch of resident synthetic inputs: the route preprocessing runs once per step
and both calls reuse it, as a training step with new routes does (the mask
built once per step in the NeMo AutoModel "flex_qsa" page), and everything
else of the full calls (delta, casts, reductions) runs inside the timed region
(the cuDNN Frontend QSA page's "Support and execution" section benchmarks the
full call). `--plain` times qsa_forward + qsa_backward instead, each call with
its own preprocessing. Outputs, plan and workspaces are allocated before the
timed region.

Prints one JSON line:
  value      sparse TFLOP/s = (4 + 10) * Hq * 256 * nnz / step time (wall clock
             over the timed steps), with nnz the number of distinct valid
             (query, key) pairs of the routes
  roofline   the longest-running kernel, on its counted work: forward 4d, dQ 6d
             (S, dP, dQ), dK/dV 4d (dV, dK; its S and dP are recomputed and
             counted once, in dQ) FLOP per (pair, head), against the dense bf16
             MFMA peak; and its HBM bytes (calibrated rocprofv3 FETCH_SIZE +
             WRITE_SIZE from the committed summary, null once the kernels
             changed) per average launch time against 8 TB/s. `bound` is the
             larger of the two fractions. Gathered kernels also report
             `gather`: their staged bytes per unit of work (1 KB of K/V per
             pair in the forward and dQ, 12 KB of Q/dO per (query, key tile)
             in dK/dV) per launch time, against the staging rate a
             direct-to-LDS probe of the same access shape reaches from L2
             (measured in the same run)
  cpu_baseline  the FP64 oracle (forward + full backward) on a bounded sample
             of the same workload, on all of this host's cores, scaled to
             TFLOP/s
"""
from __future__ import annotations

import argparse
import math
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

# Counted FLOP per (distinct valid pair, query head), by kernel: the method's
# forward (S = QK^T, O = PV) and its five backward products (S, dP, dV, dK, dQ)
# each counted once. The dK/dV kernels recompute S and dP (executed 8d), which
# the dQ kernels have already been credited with. Which pairs each kernel
# computes: "partial" = pairs outside full 128 x 128 tiles (gathered kernels),
# "full" = pairs inside them (dense kernels).
FLOP_PER_PAIR_HEAD = {
    "forward": 4 * 256,        # S = QK^T and O = PV
    "forward_dense": 4 * 256,
    "dq": 6 * 256,             # S, dP = dO V^T, dQ = dS K
    "dq_dense": 6 * 256,
    "dkdv": 4 * 256,           # dV = P^T dO, dK = dS^T Q
    "dkdv_dense": 4 * 256,
}
EXECUTED_PER_PAIR_HEAD = dict(FLOP_PER_PAIR_HEAD, dkdv=8 * 256, dkdv_dense=8 * 256)
# Staged bytes per unit of work of the gathered kernels: K and V rows (512 B
# each) per (query, key) pair; Q and dO rows (12 heads x 512 B each) per
# (query, partial 128-key tile).
GATHER_UNIT = {"forward": ("pair", 1024, 512), "dq": ("pair", 1024, 512),
               "dkdv": ("query_keytile", 12 * 1024, 6144)}
KERNEL_PAIRS = {"forward": "partial", "forward_dense": "full", "dq": "partial",
                "dq_dense": "full", "dkdv": "partial", "dkdv_dense": "full"}
COUNTED_FWD = 4 * 256
COUNTED_BWD = 10 * 256
FWD_STAGES = ["preprocess_fwd", "forward", "forward_dense"]
BWD_STAGES = ["preprocess_bwd", "delta", "dq", "dq_dense", "dkdv", "dkdv_dense", "dkdv_reduce"]
# Stage 0 of the planned calls only resets the walk clocks.
FWD_STAGES_PLANNED = ["reset_fwd"] + FWD_STAGES[1:]
BWD_STAGES_PLANNED = ["reset_bwd"] + BWD_STAGES[1:]


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


def partial_tile_hits(routes: np.ndarray, Sq: int, Skv: int) -> int:
    """(query row, key tile) pairs where the row selects a key of the tile and the
    tile is not full: the units of the gathered dK/dV."""
    B = routes.shape[0]
    nQT, nKT = (Sq + 127) // 128, (Skv + 127) // 128
    total = 0
    for b in range(B):
        r = routes[b]
        hit = np.zeros((Sq, nKT), bool)
        cnt = np.zeros((nQT, nKT), np.int64)
        for a in range(0, Sq, 1024):
            c = r[a:a + 1024].astype(np.int64)
            s = np.sort(np.where((c >= 0) & (c < Skv), c, -1), axis=-1)
            keep = s >= 0
            keep[:, 1:] &= s[:, 1:] != s[:, :-1]
            rows = np.broadcast_to(np.arange(a, a + c.shape[0])[:, None], s.shape)
            hit[rows[keep], s[keep] // 128] = True
            np.add.at(cnt, (rows[keep] // 128, s[keep] // 128), 1)
        full = cnt == 128 * 128
        hit &= ~full[np.arange(Sq) // 128]
        total += int(hit.sum())
    return total


TRAFFIC_SOURCES = ("token_indexed_sparse_amd/csrc/common.h", "token_indexed_sparse_amd/csrc/bwd.hip",
                   "token_indexed_sparse_amd/csrc/fwd.hip", "token_indexed_sparse_amd/csrc/dense.hip")


# Sources of the selector's kernels, for the same check on its summary.
SELECT_SOURCES = ("token_indexed_sparse_amd/csrc/common.h",
                  "token_indexed_sparse_amd/csrc/select.hip")


def measured_traffic(workload: str, kernel: str, sources=TRAFFIC_SOURCES):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE) from the
    committed rocprofv3 summary, or None if there is none or the kernels changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
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


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, wl, nnz_row: np.ndarray, seconds: float) -> dict:
    """The oracle (forward + full backward of a sample of query rows), timed on all
    host cores (its row loop is split over OpenMP threads)."""
    import oracle
    P = oracle.Problem(inp.q, inp.k, inp.v, inp.routes, wl.scale, inp.grad_out)
    threads = oracle.num_threads()
    rng = np.random.default_rng(0)
    rows_all = np.nonzero(nnz_row > 0)[0]

    def timed(count):
        rows = np.sort(rng.choice(rows_all, count, replace=False))
        t = time.perf_counter()
        P.backward_rows(rows)
        return rows, time.perf_counter() - t

    # Calibrate on four rows per thread, size the sample to the time budget, and
    # if that sample still ran under half the budget (a first call pays thread
    # start-up), size it again from its own time.
    n = min(4 * threads, len(rows_all))
    rows, dt = timed(n)
    for _ in range(2):
        if dt >= 0.5 * seconds or n >= len(rows_all):
            break
        n = int(max(threads, min(len(rows_all), n * seconds / max(dt, 1e-9))))
        rows, dt = timed(n)
    flop = (COUNTED_FWD + COUNTED_BWD) * wl.Hq * float(nnz_row[rows].sum())
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"forward + full backward (dq and the rows' dk/dv contributions) of {n} "
                      f"random query rows of {wl.name} ({int(nnz_row[rows].sum())} pairs), "
                      f"FP64 C oracle, {threads} OpenMP threads, {dt:.1f} s",
            "nproc": os.cpu_count(), "cpu_model": host_cpu_model()}


def gather_ceiling(torch, lib, hip, stream, row_bytes: int, footprint_bytes: int,
                   n_items: int = 1 << 22, rows=None) -> float:
    """Staging rate (GB/s) of the direct-to-LDS probe: rows of `row_bytes` drawn
    uniformly from a footprint of `footprint_bytes` (or the sequence `rows`); the
    best over the probe's launch shapes (waves per work group and LDS ring per
    wave) and work-group counts."""
    dev = torch.device("cuda:0")
    per_item = 2 if row_bytes == 512 else 1
    if rows is not None:
        # a given row sequence (two rows per item), over rows 0 .. max + 1
        nrows = int(rows.max()) + 1
        n_items = len(rows) // per_item
        idx = torch.from_numpy(rows[:n_items * per_item]).to(dev)
    else:
        nrows = max(2, footprint_bytes // row_bytes)
        g = torch.Generator(device="cpu").manual_seed(7)
        idx = torch.randint(0, nrows, (n_items * per_item,), generator=g,
                            dtype=torch.int32).to(dev)
    src = torch.zeros(nrows * row_bytes, dtype=torch.uint8, device=dev)
    ev = Events(hip, 2)
    lib.qsa_bench_gather.restype = ctypes.c_int
    lib.qsa_bench_gather.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p]

    def run(shape, blocks):
        st = lib.qsa_bench_gather(src.data_ptr(), src.numel(), idx.data_ptr(), idx.numel(),
                                  row_bytes, blocks, shape, stream)
        assert st == 0, st

    best = None
    # launch shapes x work-group counts (many short runs per wave, or one or two
    # resident work groups per CU with long runs)
    for shape in range(4):
        for blocks in (8192, 1024, 512, 256):
            run(shape, blocks)
            torch.cuda.synchronize()
            for _ in range(3):
                hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), ctypes.c_void_p(stream))
                run(shape, blocks)
                hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), ctypes.c_void_p(stream))
                torch.cuda.synchronize()
                ms = ev.elapsed(0, 1)
                best = ms if best is None else min(best, ms)
    item_bytes = 1024 if row_bytes == 512 else row_bytes  # two 512 B rows, or one 6 KB row
    return n_items * item_bytes / (best * 1e-3) / 1e9


def doc_causal_step(torch, qsa, hip, stream, wl, n_docs: int = 4, steps: int = 3) -> dict:
    """Causal attention within documents (the dense comparison workload): the same
    token count and heads as the metric's workload, `n_docs` documents at seeded cut
    points, one step = qsa_doc_plan_build + planned forward + planned backward,
    timed with HIP events; sparse TFLOP/s counted like the metric (14 * Hq * 256 per
    (query, key) pair)."""
    T = wl.Sq
    rng = np.random.default_rng(1000 + n_docs)
    cuts = np.sort(rng.choice(np.arange(1, T), n_docs - 1, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int64)
    ids = np.zeros(T, np.int32)
    for n, s0 in enumerate(starts):
        ids[s0:] = n + 1
    lens = np.diff(np.concatenate([starts, [T]]))
    pairs = int((lens * (lens + 1) // 2).sum())
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(11)

    def rnd(*shape):
        return torch.randn(*shape, generator=g).to(torch.bfloat16).to(dev)

    q, k, v, go = rnd(1, T, wl.Hq, 256), rnd(1, T, wl.Hkv, 256), rnd(1, T, wl.Hkv, 256), \
        rnd(1, T, wl.Hq, 256)
    qd = torch.from_numpy(ids[None]).to(dev)
    plan = qsa.doc_plan_build(qd, qd, Hkv=wl.Hkv)
    out, out32, lse = qsa.forward_planned(plan, q, k, v, wl.scale)
    dq, dk, dv = qsa.backward_planned(plan, go, q, k, v, out32, lse, wl.scale)
    torch.cuda.synchronize()
    ev = Events(hip, 4)
    times = []
    for _ in range(steps):
        hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), ctypes.c_void_p(stream))
        qsa.doc_plan_build(qd, qd, Hkv=wl.Hkv, plan_mem=plan.mem)
        hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), ctypes.c_void_p(stream))
        qsa.forward_planned(plan, q, k, v, wl.scale, out=out, out_fp32=out32, lse=lse)
        hip.hipEventRecord(ctypes.c_void_p(ev.ev[2]), ctypes.c_void_p(stream))
        qsa.backward_planned(plan, go, q, k, v, out32, lse, wl.scale, dq=dq, dk=dk, dv=dv)
        hip.hipEventRecord(ctypes.c_void_p(ev.ev[3]), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        times.append([ev.elapsed(0, 1), ev.elapsed(1, 2), ev.elapsed(2, 3)])
    t = np.median(np.array(times), axis=0)
    ms = float(t.sum())
    return {"workload": f"doc_causal_t{T}_{n_docs}docs_12q{wl.Hkv}kv", "T": T,
            "documents": n_docs, "pairs": pairs, "ms_per_step": ms,
            "plan_ms": float(t[0]), "forward_ms": float(t[1]), "backward_ms": float(t[2]),
            "tflops": (COUNTED_FWD + COUNTED_BWD) * wl.Hq * pairs / (ms * 1e-3) / 1e12,
            "steps": steps, "note": "median of the timed steps (HIP events), after one warm-up"}


def select_step(torch, qsa, lib, hip, stream, T: int, top_k: int, steps: int = 5) -> dict:
    """Block selector at the metric workload's token count: T queries of one sequence,
    T / 4 compressed blocks, 64 indexer heads of width 128, top_k blocks per query
    (qsa_select_timed: stage 0 the MFMA scores, stage 1 the top-k and the block and
    route outputs). Seeded normal inputs generated on the GPU. Returns the figures
    and, under "_routes", the selected route rows."""
    NB, H, D = T // 4, 64, 128
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(21)
    qi = torch.randn((1, T, H, D), generator=gen, device=dev).to(torch.bfloat16)
    kb = torch.randn((1, NB, D), generator=gen, device=dev).to(torch.bfloat16)
    sd = qsa.select_dims(qi, kb, top_k)
    ws = torch.empty(lib.qsa_select_workspace_bytes(ctypes.byref(sd)), dtype=torch.uint8,
                     device=dev)
    blocks = torch.empty((1, T, top_k), dtype=torch.int32, device=dev)
    routes = torch.empty((1, T, 4 * top_k + 4), dtype=torch.int32, device=dev)
    V, F, S, I32 = ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t, ctypes.c_int32
    lib.qsa_select_timed.restype = ctypes.c_int
    lib.qsa_select_timed.argtypes = [ctypes.POINTER(qsa.SelectDims)] + [V] * 4 + [F] + \
        [V] * 4 + [S, V, V, I32]
    scale = 1.0 / math.sqrt(D)

    def call(e=None):
        st = lib.qsa_select_timed(ctypes.byref(sd), qi.data_ptr(), kb.data_ptr(), None, None,
                                  scale, blocks.data_ptr(), routes.data_ptr(), None,
                                  ws.data_ptr(), ws.numel(), stream,
                                  ctypes.cast(e.ev, ctypes.c_void_p) if e else None,
                                  3 if e else 0)
        assert st == 0, st

    call()
    torch.cuda.synchronize()
    evs = [Events(hip, 3) for _ in range(steps)]
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    t = np.median(np.array([[e.elapsed(0, 1), e.elapsed(1, 2)] for e in evs]), axis=0)
    score_ms, topk_ms = float(t[0]), float(t[1])
    pairs = int(np.minimum(np.arange(T, dtype=np.int64) // 4, NB).sum())
    flop = 2 * H * D * pairs
    tflops = flop / (score_ms * 1e-3) / 1e12
    score_bytes = T * H * D * 2 + NB * D * 2 + 4 * pairs
    topk_bytes = 4 * pairs + 4 * T * top_k + 4 * T * (4 * top_k + 4)
    topk_gbs = topk_bytes / (topk_ms * 1e-3) / 1e9
    name = f"select_t{T}_nb{NB}_h{H}_d{D}_top{top_k}"
    tr_s = measured_traffic(name, "select_scores", SELECT_SOURCES)
    tr_k = measured_traffic(name, "select_topk", SELECT_SOURCES)
    return {"workload": name, "T": T, "NB": NB,
            "H": H, "D": D, "top_k": top_k, "visible_pairs": pairs,
            "ms": score_ms + topk_ms, "steps": steps,
            "scores": {"avg_launch_ms": score_ms, "bound": "mfma", "achieved": tflops,
                       "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": tflops / PEAK_BF16_TFLOPS, "flop_per_launch": flop,
                       "algorithmic_bytes": score_bytes, "traffic": tr_s},
            "topk": {"avg_launch_ms": topk_ms, "bound": "hbm", "achieved": topk_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": topk_gbs / PEAK_HBM_GBS,
                     "algorithmic_bytes": topk_bytes, "traffic": tr_k},
            "note": "median of the timed calls (HIP events), after one warm-up; workspace "
                    "holds the scores between the two kernels",
            "_routes": routes}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_t32768_12q1kv",
                    help="workload name or index 1-5 (default: the 32k-token long-context one)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-doc-causal", action="store_true",
                    help="skip the document-causal (dense) comparison step")
    ap.add_argument("--no-select", action="store_true",
                    help="skip the block selector measurement")
    ap.add_argument("--plain", action="store_true",
                    help="time qsa_forward + qsa_backward (preprocessing in each call) instead "
                         "of one plan build and the planned calls")
    ap.add_argument("--deterministic", action="store_true",
                    help="set QSA_FLAG_DETERMINISTIC (head-first key walks, bitwise reproducible)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--calibrate-gather", action="store_true",
                    help="print the direct-to-LDS staging rates of the gather probe and exit")
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

    lib = qsa.library()
    hip = hip_runtime()
    hip.hipEventRecord.restype = ctypes.c_int
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    if args.calibrate_gather:
        rows = []
        for rb, fp in ((512, 2 << 20), (512, 32 << 20), (6144, 2 << 20), (6144, 24 << 20),
                       (6144, 384 << 20)):
            gbs = gather_ceiling(torch, lib, hip, stream, rb, fp)
            rows.append({"row_bytes": rb, "footprint_bytes": fp, "GB/s": gbs})
            print(json.dumps(rows[-1]), flush=True)
        return 0

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
    units = {"pair": pairs["partial"],
             "query_keytile": partial_tile_hits(inp.routes, wl.Sq, wl.Skv)}

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
    plain = args.plain
    if plain:
        ws_f = torch.empty(qsa.forward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(qsa.backward_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        fwd_stages, bwd_stages = FWD_STAGES, BWD_STAGES
    else:
        lib_p = qsa.library()
        ws_f = torch.empty(lib_p.qsa_forward_planned_workspace_bytes(ctypes.byref(dims)),
                           dtype=torch.uint8, device=dev)
        ws_b = torch.empty(lib_p.qsa_backward_planned_workspace_bytes(ctypes.byref(dims)),
                           dtype=torch.uint8, device=dev)
        plan_mem = torch.empty(qsa.plan_bytes(dims), dtype=torch.uint8, device=dev)
        plan = qsa.PlanStruct()
        fwd_stages, bwd_stages = FWD_STAGES_PLANNED, BWD_STAGES_PLANNED
    V, F, S, I32 = ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t, ctypes.c_int32
    lib.qsa_forward_timed.restype = ctypes.c_int
    lib.qsa_forward_timed.argtypes = [ctypes.POINTER(qsa.Dims)] + [V] * 4 + [F] + [V] * 4 + [
        S, V, V, I32]
    lib.qsa_backward_timed.restype = ctypes.c_int
    lib.qsa_backward_timed.argtypes = [ctypes.POINTER(qsa.Dims)] + [V] * 7 + [F] + [V] * 4 + [
        S, V, V, I32]
    PL = ctypes.POINTER(qsa.PlanStruct)
    lib.qsa_forward_planned_timed.restype = ctypes.c_int
    lib.qsa_forward_planned_timed.argtypes = [PL] + [V] * 3 + [F] + [V] * 4 + [S, V, V, I32]
    lib.qsa_backward_planned_timed.restype = ctypes.c_int
    lib.qsa_backward_planned_timed.argtypes = [PL] + [V] * 6 + [F] + [V] * 4 + [S, V, V, I32]
    K, W = args.steps, args.warmup
    NF, NB = len(fwd_stages), len(bwd_stages)
    fev = [Events(hip, NF + 1) for _ in range(K)]
    bev = [Events(hip, NB + 1) for _ in range(K)]
    pev = [Events(hip, 2) for _ in range(K)]

    def step(i=None):
        fe = ctypes.cast(fev[i].ev, ctypes.c_void_p) if i is not None else None
        be = ctypes.cast(bev[i].ev, ctypes.c_void_p) if i is not None else None
        nf, nb = (NF + 1, NB + 1) if i is not None else (0, 0)
        if plain:
            st = lib.qsa_forward_timed(ctypes.byref(dims), q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), routes.data_ptr(), wl.scale, out.data_ptr(),
                                       out32.data_ptr(), lse.data_ptr(), ws_f.data_ptr(),
                                       ws_f.numel(), stream, fe, nf)
            assert st == 0, st
            st = lib.qsa_backward_timed(ctypes.byref(dims), g.data_ptr(), q.data_ptr(),
                                        k.data_ptr(), v.data_ptr(), out32.data_ptr(),
                                        lse.data_ptr(), routes.data_ptr(), wl.scale,
                                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                        ws_b.data_ptr(), ws_b.numel(), stream, be, nb)
            assert st == 0, st
            return
        if i is not None:
            assert hip.hipEventRecord(pev[i].ev[0], stream) == 0
        st = lib.qsa_plan_build(ctypes.byref(dims), routes.data_ptr(), plan_mem.data_ptr(),
                                plan_mem.numel(), ctypes.byref(plan), stream)
        assert st == 0, st
        if i is not None:
            assert hip.hipEventRecord(pev[i].ev[1], stream) == 0
        st = lib.qsa_forward_planned_timed(ctypes.byref(plan), q.data_ptr(), k.data_ptr(),
                                           v.data_ptr(), wl.scale, out.data_ptr(),
                                           out32.data_ptr(), lse.data_ptr(), ws_f.data_ptr(),
                                           ws_f.numel(), stream, fe, nf)
        assert st == 0, st
        st = lib.qsa_backward_planned_timed(ctypes.byref(plan), g.data_ptr(), q.data_ptr(),
                                            k.data_ptr(), v.data_ptr(), out32.data_ptr(),
                                            lse.data_ptr(), wl.scale, dq.data_ptr(),
                                            dk.data_ptr(), dv.data_ptr(), ws_b.data_ptr(),
                                            ws_b.numel(), stream, be, nb)
        assert st == 0, st

    print(f"[bench] warmup {W}", file=sys.stderr, flush=True)
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    # The timed region: K steps of the library's calls as a user makes them
    # (their backward runs the dQ passes beside the dK/dV passes), with an event
    # pair around each step on the stream they run on.
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    sev = [Events(hip, 2) for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        assert hip.hipEventRecord(sev[i].ev[0], stream) == 0
        step()
        assert hip.hipEventRecord(sev[i].ev[1], stream) == 0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    step_each = np.array([e.elapsed(0, 1) for e in sev])
    # Then K steps of the same calls with stage events, which run every pass
    # after the previous one: each kernel's time is its own.
    print(f"[bench] stage breakdown ({K} steps, passes in sequence)", file=sys.stderr, flush=True)
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    stage_ms = {}
    if not plain:
        stage_ms["plan"] = float(np.mean([e.elapsed(0, 1) for e in pev]))
    for a, name in enumerate(fwd_stages):
        stage_ms[name] = float(np.mean([e.elapsed(a, a + 1) for e in fev]))
    for a, name in enumerate(bwd_stages):
        stage_ms[name] = float(np.mean([e.elapsed(a, a + 1) for e in bev]))
    fwd_each = np.array([e.elapsed(0, NF) for e in fev])
    bwd_each = np.array([e.elapsed(0, NB) for e in bev])
    plan_each = np.zeros(K) if plain else np.array([e.elapsed(0, 1) for e in pev])
    serial_each = plan_each + fwd_each + bwd_each
    fwd_ms = float(np.mean(fwd_each))
    bwd_ms = float(np.mean(bwd_each))
    flop_fwd = COUNTED_FWD * wl.Hq * nnz
    flop_bwd = COUNTED_BWD * wl.Hq * nnz
    value = (flop_fwd + flop_bwd) / (ms_step * 1e-3) / 1e12

    # gather ceiling: the best direct-to-LDS staging rate the probe reaches from an
    # L2-resident footprint (2 MB), over both row shapes (512-byte K/V rows two per
    # load, 6 KB Q/dO rows), launch shapes and work-group counts
    print("[bench] gather probe", file=sys.stderr, flush=True)
    ceiling = {rb: gather_ceiling(torch, lib, hip, stream, rb, 2 << 20) for rb in (512, 6144)}
    best_rb = max(ceiling, key=ceiling.get)
    gather_peak = ceiling[best_rb]
    gather_source = (f"best L2-resident staging rate of the direct-to-LDS probe ({best_rb}-byte "
                     "rows, 2 MB footprint; best of both row shapes)")

    def kernel_roofline(name):
        ms = stage_ms[name]
        flop = FLOP_PER_PAIR_HEAD[name] * wl.Hq * pairs[KERNEL_PAIRS[name]]
        tflops = flop / (ms * 1e-3) / 1e12
        traffic = measured_traffic(wl.name, name)
        r = {"kernel": name, "avg_launch_ms": ms,
             "mfma": {"achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": tflops / PEAK_BF16_TFLOPS, "counted_flop_per_launch": flop,
                      "executed_flop_per_launch":
                          EXECUTED_PER_PAIR_HEAD[name] * wl.Hq * pairs[KERNEL_PAIRS[name]]},
             "traffic": traffic}
        if traffic is not None:
            gbs = traffic / (ms * 1e-3) / 1e9
            r["hbm"] = {"achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS,
                        "note": "FETCH_SIZE counts fetches beyond L2; the last-level cache "
                                "(MALL) may serve part of them"}
        if name in GATHER_UNIT:
            unit, nbytes, rb = GATHER_UNIT[name]
            staged = nbytes * units[unit]
            gbs = staged / (ms * 1e-3) / 1e9
            r["gather"] = {"achieved": gbs, "peak": gather_peak, "unit": "GB/s",
                           "frac": gbs / gather_peak, "unit_of_work": unit,
                           "bytes_per_unit": nbytes, "units_per_launch": units[unit],
                           "staged_bytes_per_launch": staged,
                           "same_shape_probe_gbs": ceiling[rb],
                           "peak_source": gather_source}
        return r

    per_kernel = {n: kernel_roofline(n) for n in KERNEL_PAIRS}
    dom = max(KERNEL_PAIRS, key=lambda s: stage_ms[s])
    d = per_kernel[dom]
    use_hbm = "hbm" in d and d["hbm"]["frac"] > d["mfma"]["frac"]
    main_part = d["hbm"] if use_hbm else d["mfma"]
    roofline = {"bound": "hbm" if use_hbm else "mfma", "kernel": dom,
                "achieved": main_part["achieved"], "peak": main_part["peak"],
                "unit": main_part["unit"], "frac": main_part["frac"], "traffic": d["traffic"],
                "avg_launch_ms": d["avg_launch_ms"], "mfma": d["mfma"]}
    for key in ("hbm", "gather"):
        if key in d:
            roofline[key] = d[key]

    # algorithmic HBM bytes of one step (each tensor once per call; the backward
    # also writes and reads its bit-packed membership once)
    Bq = wl.B * wl.Sq * wl.Hq * wl.D
    Bk = wl.B * wl.Skv * wl.Hkv * wl.D
    mbits = wl.B * wl.Sq * (-(-wl.Skv // 128) * 128) // 8
    rt = inp.routes.nbytes
    lse_b = 4 * wl.B * wl.Hq * wl.Sq
    fwd_bytes = rt + 2 * Bq + 2 * 2 * Bk + 2 * Bq + 4 * Bq + lse_b
    bwd_bytes = (rt + 2 * mbits + 2 * Bq + 2 * 2 * Bk + 2 * Bq + 4 * Bq + lse_b + 2 * lse_b
                 + 2 * Bq + 2 * 2 * Bk)
    step_bytes = fwd_bytes + bwd_bytes - (0 if plain else rt)  # a plan reads the routes once

    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Sq": wl.Sq, "Skv": wl.Skv, "Hq": wl.Hq,
                   "Hkv": wl.Hkv, "D": wl.D, "W": wl.W, "nnz_pairs": nnz, "full_tile_pairs": nnz_full,
                   "partial_query_keytile_pairs": units["query_keytile"],
                   "flop_per_step": flop_fwd + flop_bwd, "parallelism": "single GPU",
                   "route_preprocessing": "per call" if plain else "once per step (plan)",
                   "deterministic": bool(args.deterministic)},
        "mfma_peak_frac": value / PEAK_BF16_TFLOPS,
        "step_ms_events": {"median": float(np.median(step_each)), "min": float(np.min(step_each)),
                           "mean": float(np.mean(step_each))},
        "forward_tflops": flop_fwd / (fwd_ms * 1e-3) / 1e12,
        "backward_tflops": flop_bwd / (bwd_ms * 1e-3) / 1e12,
        "stage_ms": stage_ms,
        "stage_note": "stage_ms, forward_tflops, backward_tflops and the kernel rooflines come "
                      "from a second run of the same steps with stage events, in which every "
                      "pass waits for the previous one; in the timed steps the backward runs "
                      "its dQ passes beside its dK/dV passes",
        "serial_step_ms_events": {"median": float(np.median(serial_each)),
                                  "min": float(np.min(serial_each))},
        "algorithmic_hbm_gbs": step_bytes / (ms_step * 1e-3) / 1e9,
        "gather_ceiling_gbs": {str(k): v for k, v in ceiling.items()},
        "roofline": roofline,
        "kernels": {n: {k2: v2 for k2, v2 in r.items() if k2 != "kernel"}
                    for n, r in per_kernel.items()},
    }
    if not args.no_select:
        print("[bench] block selector", file=sys.stderr, flush=True)
        sel = select_step(torch, qsa, lib, hip, stream, wl.Sq, wl.n_max)
        r_sel = sel.pop("_routes")
        if not plain and wl.B == 1 and wl.Sq == wl.Skv and r_sel.shape == routes.shape:
            # plan build + forward + backward over the selector's routes
            sel_pairs = int((r_sel >= 0).sum().item())
            times = []
            for i in range(4):
                hip.hipEventRecord(ctypes.c_void_p(pev[0].ev[0]), ctypes.c_void_p(stream))
                st = lib.qsa_plan_build(ctypes.byref(dims), r_sel.data_ptr(), plan_mem.data_ptr(),
                                        plan_mem.numel(), ctypes.byref(plan), stream)
                assert st == 0, st
                st = lib.qsa_forward_planned_timed(ctypes.byref(plan), q.data_ptr(), k.data_ptr(),
                                                   v.data_ptr(), wl.scale, out.data_ptr(),
                                                   out32.data_ptr(), lse.data_ptr(),
                                                   ws_f.data_ptr(), ws_f.numel(), stream, None, 0)
                assert st == 0, st
                st = lib.qsa_backward_planned_timed(ctypes.byref(plan), g.data_ptr(),
                                                    q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                    out32.data_ptr(), lse.data_ptr(), wl.scale,
                                                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                                    ws_b.data_ptr(), ws_b.numel(), stream, None,
                                                    0)
                assert st == 0, st
                hip.hipEventRecord(ctypes.c_void_p(pev[0].ev[1]), ctypes.c_void_p(stream))
                torch.cuda.synchronize()
                if i:
                    times.append(pev[0].elapsed(0, 1))
            att_ms = float(np.median(times))
            sel["attention_on_selected"] = {
                "pairs": sel_pairs, "ms_per_step": att_ms,
                "tflops": (COUNTED_FWD + COUNTED_BWD) * wl.Hq * sel_pairs / (att_ms * 1e-3) / 1e12,
                "select_plus_step_ms": att_ms + sel["ms"],
                "note": "plan build + forward + backward of the metric's attention shapes over "
                        "the route rows the selector produced (median of 3 after a warm-up)"}
        del r_sel
        res["select"] = sel
    if not args.no_doc_causal:
        print("[bench] document-causal comparison", file=sys.stderr, flush=True)
        res["doc_causal"] = doc_causal_step(torch, qsa, hip, stream, wl)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, wl, nnz_row, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
