"""Benchmark of the SLiM compressed linear layer on one MI355X.

Headline (one JSON line on stdout): slim_linear on the LLaMA-2-7B q_proj
shape at decode, M = 1 token (X [1, 4096], W [4096, 4096] int4 g128 2:4,
adapter rank 416), as HBM GB/s of algorithmic bytes.  A step is one
slim_linear call on one token batch; every call reads a different, already
HBM-resident buffer set (X, packed W, L, R, Y) from a pool of >= 1 GiB, so
the ~256 MB last-level cache cannot serve repeated calls.

Also reported in the same line: M = 16 decode, the M = 2048 down_proj prefill
(TFLOP/s), a dense fp16 torch.matmul of each shape, the one-shot pack, the
roofline of the dominant kernel and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "2:4-int4+low-rank linear: µs/call, HBM GB/s (M=1), TFLOP/s (M=2048)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
POOL_BYTES = 1 << 30


def alg_bytes(M, N, K, r):
    return N * K // 4 + N * K // 8 + N * K // 64 + 2 * M * K + 2 * K * r + 2 * r * N + 2 * M * N


def alg_flops(M, N, K, r):
    return M * N * K + 2 * M * K * r + 2 * M * r * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class LayerPool:
    """Distinct, seeded, device-resident buffer sets for one layer shape."""

    def __init__(self, torch, slim, M, N, K, r, min_bytes, seed=1234, max_sets=256):
        self.M, self.N, self.K, self.r = M, N, K, r
        per = alg_bytes(M, N, K, r)
        self.nsets = max(2, min(max_sets, math.ceil(min_bytes / per)))
        g = torch.Generator(device="cuda")
        self.sets = []
        for i in range(self.nsets):
            g.manual_seed(seed + i)
            W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
            w = slim.pack(W)
            del W
            X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).half()
            L = (torch.randn((r, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).half()  # L^T
            R = (torch.randn((N, r), generator=g, device="cuda", dtype=torch.float32) * 0.02).half()  # R^T
            Y = torch.empty((M, N), device="cuda", dtype=torch.float16)
            self.sets.append((X, w, L, R, Y))
        self.ws = slim.workspace(M, N, K, r)
        torch.cuda.synchronize()

    def call(self, slim, i):
        X, w, L, R, Y = self.sets[i % self.nsets]
        slim.slim_linear(X, w.values, w.meta, w.scales, L, R, Y, self.ws)


def time_loop(torch, fn, steps, warmup, graph=True):
    """ms per call of fn over `steps` calls on the current stream.

    With graph=True the calls are captured once into a HIP graph and the
    timed region is one replay, so host-side launch overhead (Python, ctypes)
    does not hide the GPU time; the events bracket the replay on the stream
    the kernels run on."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if not graph:
        start.record(stream)
        for i in range(steps):
            fn(warmup + i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(steps):
                fn(warmup + i)
    stream.wait_stream(cap)
    g.replay()                      # untimed replay: first-launch costs
    torch.cuda.synchronize()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / steps


def bench_slim(torch, slim, M, N, K, r, steps, warmup, reps=5, eager=False):
    pool = LayerPool(torch, slim, M, N, K, r, POOL_BYTES)
    times = [time_loop(torch, lambda i: pool.call(slim, i), steps, warmup) for _ in range(reps)]
    if eager:
        times_eager = time_loop(torch, lambda i: pool.call(slim, i), steps, warmup, graph=False)
    del pool
    torch.cuda.empty_cache()
    return (times, times_eager) if eager else times


def bench_dense(torch, M, N, K, steps, warmup, reps=3):
    per = 2 * N * K + 2 * M * K + 2 * M * N
    n = max(2, min(64, math.ceil(POOL_BYTES / per)))
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    Ws = [torch.randn((N, K), generator=g, device="cuda", dtype=torch.float16) for _ in range(n)]
    Xs = [torch.randn((M, K), generator=g, device="cuda", dtype=torch.float16) for _ in range(n)]
    Ys = [torch.empty((M, N), device="cuda", dtype=torch.float16) for _ in range(n)]

    def fn(i):
        j = i % n
        torch.matmul(Xs[j], Ws[j].t(), out=Ys[j])

    try:
        times = [time_loop(torch, fn, steps, warmup) for _ in range(reps)]
    except RuntimeError:            # library refused graph capture: time it eagerly
        times = [time_loop(torch, fn, steps, warmup, graph=False) for _ in range(reps)]
    del Ws, Xs, Ys
    torch.cuda.empty_cache()
    return statistics.median(times)


def bench_pack(torch, slim, N, K, steps, warmup):
    n = max(2, min(16, math.ceil(POOL_BYTES / (4 * N * K))))
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    Ws = [torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02 for _ in range(n)]
    outs = [slim.pack(W) for W in Ws]

    def fn(i):
        j = i % n
        o = outs[j]
        slim.slim_pack(Ws[j], o.values, o.meta, o.scales)

    t = time_loop(torch, fn, steps, warmup)
    del Ws, outs
    torch.cuda.empty_cache()
    return t


def cpu_baseline(budget_s=12.0):
    """The CPU oracle as it stands, on q_proj M=1: repeat for ~budget_s."""
    import numpy as np
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    case = wl.QPROJ
    inp = wl.make_inputs(case)
    v, m, s = oracle.pack(inp.W)
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.linear(inp.X, v, m, s, inp.L, inp.R)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / calls
    gbs = alg_bytes(case.M, case.N, case.K, case.r) / per / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"{calls} oracle.linear calls on q_proj M=1 (4096x4096, r=416) in {el:.1f} s, "
                      f"{per * 1e3:.1f} ms/call; numpy fp64, BLAS threads={blas_threads}, "
                      f"host cpu_count={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling)")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this build has no "
              f"multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    slim._lib.load()

    M, N, K, r = 1, 4096, 4096, 416
    ms_list, ms_eager = bench_slim(torch, slim, M, N, K, r, args.steps, args.warmup, eager=True)
    ms = statistics.median(ms_list)
    nbytes = alg_bytes(M, N, K, r)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"q_proj M=1: {ms * 1e3:.2f} us/call ({[round(t * 1e3, 2) for t in ms_list]}), {gbs:.0f} GB/s")

    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "q_proj decode: X[1,4096] fp16, W[4096,4096] int4 g128 2:4, r=416",
                   "M": M, "N": N, "K": K, "r": r, "group": 128},
        "us_per_call": round(ms * 1e3, 3),
        "timing": "HIP graph of `steps` calls replayed once between events; eager_us_per_call is the same "
                  "loop launched call by call from Python (host-bound)",
        "eager_us_per_call": round(ms_eager * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "per_launch_bytes": nbytes, "note": "whole slim_linear call (all its launches)"},
    }
    if not args.quick:
        extra = {}
        for (name, mM, nN, kK) in (("q_proj_M16", 16, 4096, 4096), ("gate_up_M16", 16, 11008, 4096)):
            t = statistics.median(bench_slim(torch, slim, mM, nN, kK, r, args.steps, args.warmup, reps=3))
            b = alg_bytes(mM, nN, kK, r)
            extra[name] = {"us_per_call": round(t * 1e3, 3), "GB/s": round(b / (t * 1e-3) / 1e9, 1),
                           "hbm_frac": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"{name}: {t * 1e3:.2f} us/call")
        Mp, Np, Kp = 2048, 4096, 11008
        tp = statistics.median(bench_slim(torch, slim, Mp, Np, Kp, r, max(3, args.steps // 40), 2, reps=1))
        fl = alg_flops(Mp, Np, Kp, r)
        extra["down_M2048"] = {"us_per_call": round(tp * 1e3, 2), "TFLOP/s": round(fl / (tp * 1e-3) / 1e12, 2),
                               "mfma_frac": round(fl / (tp * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4)}
        log(f"down M=2048: {tp * 1e3:.1f} us/call")
        dense = {}
        for (name, mM, nN, kK) in (("q_proj_M1", 1, 4096, 4096), ("q_proj_M16", 16, 4096, 4096),
                                   ("gate_up_M16", 16, 11008, 4096), ("down_M2048", 2048, 4096, 11008)):
            t = bench_dense(torch, mM, nN, kK, max(10, args.steps // 4), 5)
            dense[name] = {"us_per_call": round(t * 1e3, 3)}
        extra["dense_fp16_matmul"] = dense
        extra["speedup_vs_dense_M1"] = round(dense["q_proj_M1"]["us_per_call"] / (ms * 1e3), 3)
        tpk = bench_pack(torch, slim, 4096, 4096, 50, 5)
        extra["pack_q_proj"] = {"us_per_call": round(tpk * 1e3, 2),
                                "GB/s": round(4096 * 4096 * (4 + 25 / 64) / (tpk * 1e-3) / 1e9, 1)}
        out["extra"] = extra
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
