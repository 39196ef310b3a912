"""Benchmark of the SLiM compressed linear layer on one MI355X.

Headline (one JSON line on stdout): slim_linear on the LLaMA-2-7B q_proj
shape at decode, M = 1 token (X [1, 4096], W [4096, 4096] int4 g128 2:4,
adapter rank 416), as HBM GB/s of algorithmic bytes.  A step is one
slim_linear call on one token batch; every call reads a different, already
HBM-resident buffer set (X, packed W, L, R, Y) from a pool of >= 1 GiB, so
the ~256 MB last-level cache cannot serve repeated calls.

Also reported in the same line: the LLaMA-2-7B decoder-block sweep (q/k/v/o,
gate/up and down shapes at M = 1, 16, 256, 2048 tokens) with a dense fp16
torch.matmul of each shape, the one-shot pack, the roofline of the timed call
and the CPU oracle timed on a bounded sample.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
  python bench.py --profile            # short headline run + a 256 MiB copy, for rocprofv3
  python bench.py --profile --transposed --shape 1 N K 0   # slim_pack_transposed of an N x K weight
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR
        # reduce two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
        # `--profile` to profiles/traffic_q_proj_M1.json (HBM bytes per call,
        # scaled by what the counters read for the copy of known size)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
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
COPY_CALIB_BYTES = 256 << 20   # plain device-to-device copy used to scale the byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q_proj_M1.json")
SWEEP_SHAPES = (("qkvo", 4096, 4096), ("gate_up", 11008, 4096), ("down", 4096, 11008))
SWEEP_M = (1, 16, 256, 2048)
HEADLINE = (1, 4096, 4096, 416)


def alg_bytes(M, N, K, r):
    return N * K // 4 + N * K // 8 + N * K // 64 + 2 * M * K + 2 * K * r + 2 * r * N + 2 * M * N


def alg_flops(M, N, K, r):
    return M * N * K + 2 * M * K * r + 2 * M * r * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def t_roof_us(M, N, K, r):
    """Lower bound on the call time from HBM bytes and fp16 MFMA FLOPs."""
    return max(alg_bytes(M, N, K, r) / (HBM_PEAK_GBS * 1e9), alg_flops(M, N, K, r) / (FP16_PEAK_TFLOPS * 1e12)) * 1e6


# Sources of the code the headline (one-token decode) shape runs: the decode
# kernels, the dispatcher and the ABI.  The prefill, generic and pack kernels
# never run at that shape, so their edits leave its byte counters valid.
HEADLINE_SOURCES = ("sparse_int4_gemm_amd/csrc/dispatch.cpp", "sparse_int4_gemm_amd/csrc/internal.hpp",
                    "sparse_int4_gemm_amd/csrc/mfma_util.hpp", "sparse_int4_gemm_amd/csrc/slim_api.cpp",
                    "sparse_int4_gemm_amd/csrc/linear_decode.hip", "include/slim.h")


def kernel_source_hash():
    """Hash of the sources the headline shape runs: byte counters taken on
    other sources no longer describe the kernels that run."""
    h = hashlib.sha256()
    for rel in HEADLINE_SOURCES:
        h.update(os.path.basename(rel).encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def alg_bytes_qa(M, N, K, r):
    """Bytes of one call with int4 adapter factors (codes + fp16 group scales:
    groups of 128 along K for Lt, of 32 along r for Rt)."""
    return (N * K // 4 + N * K // 8 + N * K // 64 + 2 * M * K + K * r // 2 + (K // 128) * r * 2
            + N * r // 2 + (r // 32) * N * 2 + 2 * M * N)


class QALayerPool:
    """LayerPool with quantised adapters (slim_linear_qa)."""

    def __init__(self, torch, slim, M, N, K, r, min_bytes, seed=4321, max_sets=256):
        self.M, self.N, self.K, self.r = M, N, K, r
        self.nsets = max(2, min(max_sets, math.ceil(min_bytes / alg_bytes_qa(M, N, K, r))))
        g = torch.Generator(device="cuda")
        self.sets = []
        for i in range(self.nsets):
            g.manual_seed(seed + i)
            W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
            w = slim.pack(W)
            del W
            X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).half()
            Lt = torch.randn((r, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
            Rt = torch.randn((N, r), generator=g, device="cuda", dtype=torch.float32) * 0.02
            qa = slim.pack_adapters(Lt, Rt)
            del Lt, Rt
            Y = torch.empty((M, N), device="cuda", dtype=torch.float16)
            self.sets.append((X, w, qa, Y))
        self.ws = slim.workspace_qa(M, N, K, r)
        torch.cuda.synchronize()

    def call(self, slim, i):
        X, w, qa, Y = self.sets[i % self.nsets]
        slim.slim_linear_qa(X, w.values, w.meta, w.scales, qa.lq, qa.ls, qa.rq, qa.rs, qa.r, Y, self.ws)


def bench_qa(torch, slim, r, steps, fp16_sweep):
    """slim_linear_qa on the decode and prefill ends of the sweep, beside the
    same shapes with fp16 adapters."""
    res = {}
    for (name, N, K, M) in (("qkvo", 4096, 4096, 1), ("down", 4096, 11008, 1), ("qkvo", 4096, 4096, 16),
                            ("down", 4096, 11008, 2048)):
        pool = QALayerPool(torch, slim, M, N, K, r, POOL_BYTES)
        t = statistics.median([time_loop(torch, lambda i: pool.call(slim, i), steps, 5) for _ in range(3)])
        del pool
        torch.cuda.empty_cache()
        us = t * 1e3
        b = alg_bytes_qa(M, N, K, r)
        key = f"{name}@M{M}"
        res[key] = {"us_per_call": round(us, 3), "bytes": b, "GB/s": round(b / us / 1e3, 1),
                    "fp16_adapter_us": fp16_sweep.get(key, {}).get("us_per_call"),
                    "fp16_adapter_bytes": alg_bytes(M, N, K, r)}
        log(f"quantised adapters {key}: {us:.2f} us")
    return res


class A8LayerPool:
    """LayerPool with an 8-bit input: per set the int8 codes and fp16 token
    scales of X (made by slim_quantize_input from an fp16 X), and X itself
    for the quantiser's own timing."""

    def __init__(self, torch, slim, M, N, K, r, min_bytes, seed=5678, max_sets=256):
        self.M, self.N, self.K, self.r = M, N, K, r
        self.nsets = max(2, min(max_sets, math.ceil(min_bytes / alg_bytes_a8(M, N, K, r))))
        g = torch.Generator(device="cuda")
        self.sets = []
        for i in range(self.nsets):
            g.manual_seed(seed + i)
            W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
            w = slim.pack(W)
            del W
            X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).half()
            q, s = slim.quantize_input(X)
            L = (torch.randn((r, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).half()
            R = (torch.randn((N, r), generator=g, device="cuda", dtype=torch.float32) * 0.02).half()
            Y = torch.empty((M, N), device="cuda", dtype=torch.float16)
            self.sets.append((X, q, s, w, L, R, Y))
        self.ws = torch.zeros(slim.slim_linear_a8_workspace_bytes(M, N, K, r), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def call(self, slim, i):
        X, q, s, w, L, R, Y = self.sets[i % self.nsets]
        slim.slim_linear_a8(q, s, w.values, w.meta, w.scales, L, R, Y, self.ws)

    def quantize(self, slim, i):
        X, q, s, w, L, R, Y = self.sets[i % self.nsets]
        slim.slim_quantize_input(X, q, s)


def alg_bytes_a8(M, N, K, r):
    """Bytes of one slim_linear_a8 call: the input is M K int8 codes and M fp16 scales."""
    return alg_bytes(M, N, K, r) - M * K + 2 * M


def bench_a8(torch, slim, r, steps, fp16_sweep):
    """slim_linear_a8 (8-bit input) on decode and prefill shapes, beside the
    fp16-input layer of the same shape, and the per-token quantiser."""
    res = {}
    for (name, N, K, M, rr) in (("qkvo", 4096, 4096, 1, r), ("qkvo", 4096, 4096, 16, r), ("qkvo", 4096, 4096, 2048, r),
                                ("down", 4096, 11008, 2048, r), ("down", 4096, 11008, 2048, 0)):
        pool = A8LayerPool(torch, slim, M, N, K, rr, POOL_BYTES)
        t = statistics.median([time_loop(torch, lambda i: pool.call(slim, i), steps, 5) for _ in range(3)])
        tq = statistics.median([time_loop(torch, lambda i: pool.quantize(slim, i), steps, 5) for _ in range(3)])
        del pool
        torch.cuda.empty_cache()
        us, usq = t * 1e3, tq * 1e3
        key = f"{name}@M{M}" + ("" if rr == r else f"_r{rr}")
        res[key] = {"us_per_call": round(us, 3), "GB/s": round(alg_bytes_a8(M, N, K, rr) / us / 1e3, 1),
                    "TFLOP/s": round(alg_flops(M, N, K, rr) / us / 1e6, 2),
                    "fp16_input_us": fp16_sweep.get(key, {}).get("us_per_call"),
                    "quantize_input_us": round(usq, 3)}
        log(f"8-bit input {key}: {us:.2f} us (quantiser {usq:.2f} us)")
    return res


def alg_bytes_hybrid(M, N, K, r, dense_frac):
    """Bytes of one slim_linear_hybrid call: the 2:4 call's plus the second
    pair of codes of the dense tiles (N K/4 bytes at all-dense) and the tile
    flags (4 bytes per 16 x 128 tile)."""
    return alg_bytes(M, N, K, r) + int(dense_frac * N * K // 4) + (N // 16) * (K // 128) * 4


def alg_flops_hybrid(M, N, K, r, dense_frac):
    return alg_flops(M, N, K, r) + int(dense_frac * M * N * K)


class HybridLayerPool:
    """LayerPool with hybrid dense / 2:4 weights: a seeded random tile mask
    with the given fraction of dense tiles per buffer set."""

    def __init__(self, torch, slim, M, N, K, r, dense_frac, min_bytes, seed=2468, max_sets=256):
        self.M, self.N, self.K, self.r = M, N, K, r
        self.nsets = max(2, min(max_sets, math.ceil(min_bytes / alg_bytes_hybrid(M, N, K, r, dense_frac))))
        g = torch.Generator(device="cuda")
        self.sets = []
        for i in range(self.nsets):
            g.manual_seed(seed + i)
            W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
            dense = (torch.rand(((N + 15) // 16, K // 128), generator=g, device="cuda") < dense_frac).to(torch.int32)
            w = slim.pack_hybrid(W, dense)
            del W
            X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).half()
            L = (torch.randn((r, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).half()
            R = (torch.randn((N, r), generator=g, device="cuda", dtype=torch.float32) * 0.02).half()
            Y = torch.empty((M, N), device="cuda", dtype=torch.float16)
            self.sets.append((X, w, L, R, Y))
        self.ws = slim.workspace(M, N, K, r)
        torch.cuda.synchronize()

    def call(self, slim, i):
        X, w, L, R, Y = self.sets[i % self.nsets]
        slim.slim_linear_hybrid(X, w.values, w.meta, w.scales, w.dvalues, w.dense, L, R, Y, self.ws)


def bench_hybrid(torch, slim, r, steps, fp16_sweep):
    """slim_linear_hybrid at 0, 25, 50 and 100% dense tiles, on q_proj at one
    token and down_proj at 2048 tokens, beside slim_linear (all 2:4) and the
    dense fp16 matmul of the sweep."""
    res = {}
    for (name, N, K, M) in (("qkvo", 4096, 4096, 1), ("down", 4096, 11008, 2048)):
        key = f"{name}@M{M}"
        row = {"slim_linear_us": fp16_sweep.get(key, {}).get("us_per_call"),
               "dense_fp16_us": fp16_sweep.get(key, {}).get("dense_fp16_us")}
        for frac in (0.0, 0.25, 0.5, 1.0):
            pool = HybridLayerPool(torch, slim, M, N, K, r, frac, POOL_BYTES)
            t = statistics.median([time_loop(torch, lambda i: pool.call(slim, i), steps, 5) for _ in range(3)])
            del pool
            torch.cuda.empty_cache()
            us = t * 1e3
            row[f"dense{int(frac * 100)}"] = {"us_per_call": round(us, 3),
                                             "GB/s": round(alg_bytes_hybrid(M, N, K, r, frac) / us / 1e3, 1),
                                             "TFLOP/s": round(alg_flops_hybrid(M, N, K, r, frac) / us / 1e6, 2)}
            log(f"hybrid {key} dense {frac:.2f}: {us:.2f} us")
        res[key] = row
    return res


def time_loop(torch, fn, steps, warmup, graph=True):
    """ms per call of fn over `steps` calls on the current stream.

    fn(i) runs call i of one continuing sequence: warmup calls 0 .. W-1, then
    calls W .. W+S-1 (untimed), then the timed calls W+S .. W+2S-1.  A pool
    cycles through its buffer sets in that order, so every call reads a set
    last touched one whole pool (>= 1 GiB) earlier, whatever the step count,
    and the ~256 MB last-level cache cannot serve it.

    With graph=True each block of S calls is captured into its own HIP graph
    and the timed region is one replay of the second, so host-side launch
    overhead (Python, ctypes) does not hide the GPU time; the events bracket
    the replay on the stream the kernels run on."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if not graph:
        for i in range(steps):
            fn(warmup + i)
        start.record(stream)
        for i in range(steps):
            fn(warmup + steps + i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps
    graphs = []
    cap = torch.cuda.Stream()
    for blk in range(2):
        g = torch.cuda.CUDAGraph()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    fn(warmup + blk * steps + i)
        stream.wait_stream(cap)
        graphs.append(g)
    graphs[0].replay()              # untimed: first-launch costs, and the calls before the timed ones
    start.record(stream)
    graphs[1].replay()
    end.record(stream)
    torch.cuda.synchronize()
    del graphs
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


def bench_pack_transposed(torch, slim, N, K, steps, warmup):
    """slim_pack_transposed over a pool of packed weights (HBM-resident
    inputs and outputs, rotated so that no call reads what the last one
    left in the caches)."""
    per = N * K * (25 / 64 + 9 / 8)
    n = max(2, min(48, math.ceil(POOL_BYTES / per)))
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    ws = []
    for _ in range(n):
        W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32) * 0.02
        ws.append(slim.pack(W))
        del W
    outs = [slim.pack_transposed(w) for w in ws]

    def fn(i):
        j = i % n
        slim.slim_pack_transposed(ws[j].values, ws[j].meta, ws[j].scales, N, K, outs[j][0], outs[j][1])

    t = time_loop(torch, fn, steps, warmup)
    del ws, outs
    torch.cuda.empty_cache()
    return t


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _timed(fn, min_s=0.5, max_calls=50):
    """Seconds per call of fn(): repeated until min_s has passed."""
    calls, t0 = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        el = time.perf_counter() - t0
        if el >= min_s or calls >= max_calls:
            return el / calls, calls


def cpu_baseline(budget_s=8.0):
    """The CPU oracle as it stands (numpy fp64, all BLAS threads).

    Headline figure: oracle.linear on q_proj M=1, repeated for ~budget_s, as
    GB/s of the call's algorithmic bytes.  Beside it: oracle.pack and
    oracle.linear separately on each configuration (tiny, q_proj M=1 and 16,
    gate/up M=16, down M=2048), and a 1-thread figure for tiny and q_proj."""
    import numpy as np  # noqa: F401
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        blas_threads = 1
    case = wl.QPROJ
    inp = wl.make_inputs(case)
    tp0 = time.perf_counter()
    v, m, s = oracle.pack(inp.W)
    pack_s = time.perf_counter() - tp0
    per, calls = _timed(lambda: oracle.linear(inp.X, v, m, s, inp.L, inp.R), budget_s, 10 ** 6)
    gbs = alg_bytes(case.M, case.N, case.K, case.r) / per / 1e9

    per_config = {}
    for c in (wl.TINY, wl.QPROJ, wl.QPROJ.with_M(16), wl.GATEUP, wl.DOWN):
        ci = wl.make_inputs(c)
        t0 = time.perf_counter()
        cv, cm, cs = oracle.pack(ci.W)
        tpk = time.perf_counter() - t0
        tl, n = _timed(lambda: oracle.linear(ci.X, cv, cm, cs, ci.L, ci.R), 0.5, 20)
        row = {"pack_s": round(tpk, 4), "linear_s": round(tl, 5), "linear_calls": n,
               "linear_GB/s": round(alg_bytes(c.M, c.N, c.K, c.r) / tl / 1e9, 4),
               "linear_GFLOP/s": round(alg_flops(c.M, c.N, c.K, c.r) / tl / 1e9, 3)}
        if c in (wl.TINY, wl.QPROJ) and threadpool_limits is not None:
            with threadpool_limits(limits=1):
                t1, _ = _timed(lambda: oracle.linear(ci.X, cv, cm, cs, ci.L, ci.R), 0.5, 10)
                t0 = time.perf_counter()
                oracle.pack(ci.W)
                row["pack_s_1thread"] = round(time.perf_counter() - t0, 4)
            row["linear_s_1thread"] = round(t1, 5)
        per_config[c.name if "@" in c.name else f"{c.name}@M{c.M}"] = row
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"{calls} oracle.linear calls on q_proj M=1 (4096x4096, r=416) in {per * calls:.1f} s, "
                      f"{per * 1e3:.1f} ms/call; numpy fp64, BLAS threads={blas_threads}, "
                      f"host cpu_count={os.cpu_count()}; oracle.pack of the 4096x4096 weight: "
                      f"{pack_s:.2f} s; per_config: one oracle.pack and >= 0.5 s of oracle.linear calls "
                      f"per configuration",
            "cpu_model": cpu_model(), "cpu_count": os.cpu_count(), "pack_s": round(pack_s, 3),
            "per_config": per_config}


def gpu_clock():
    """Current shader clock as reported by rocm-smi (best effort, text)."""
    import subprocess
    try:
        res = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        lines = [ln.strip() for ln in res.stdout.splitlines() if "sclk" in ln.lower() or "fclk" in ln.lower()
                 or "mclk" in ln.lower()]
        return "; ".join(lines)[:300] or None
    except Exception:
        return None


def traffic_from_profile(M, N, K, r, per_call_bytes):
    """HBM bytes per call from the committed counter summary, if it was taken
    on the kernel sources that are running now; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None, "no counter summary"
    if t.get("source_hash") != kernel_source_hash():
        return None, "counter summary taken on other kernel sources"
    if tuple(t.get("shape", ())) != (M, N, K, r):
        return None, "counter summary for another shape"
    return t["hbm_bytes_per_call"], (f"rocprofv3 FETCH_SIZE x{t['fetch_scale']:.3f} + WRITE_SIZE "
                                     f"x{t['write_scale']:.3f} per call ({t['calls']} calls), scaled by a "
                                     f"{COPY_CALIB_BYTES >> 20} MiB copy; algorithmic {per_call_bytes} B")


def _pmc_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def summarize_pmc(fetch_dir, write_dir):
    """Reduce the two counter runs of `bench.py --profile` to HBM bytes per
    slim_linear call of the headline shape.  FETCH_SIZE and WRITE_SIZE are in
    KiB per dispatch; each is scaled so that the plain copy of
    COPY_CALIB_BYTES reads (writes) exactly that many bytes."""
    out = {"shape": list(HEADLINE), "source_hash": kernel_source_hash(),
           "command": "cd /tmp && rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -- python3 bench.py --profile; "
                      "rocprofv3 --pmc WRITE_SIZE -d <write_dir> -- python3 bench.py --profile; "
                      "python3 bench.py --summarize-pmc <fetch_dir> <write_dir>"}
    calls = None
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        slim_k, copy_k = {}, []
        for row in _pmc_rows(d):
            if row["Counter_Name"] != counter:
                continue
            name, v = row["Kernel_Name"], float(row["Counter_Value"])
            if "slim::" in name and "pack_kernel" not in name:
                short = name.replace("(anonymous namespace)::", "").split("(")[0]
                short = short.replace("void ", "").replace("slim::", "")
                slim_k.setdefault(short, []).append(v)
            elif "copyBuffer" in name or "copy_kernel" in name or "CopyKernel" in name:
                copy_k.append(v)
        if not copy_k or not slim_k:
            raise SystemExit(f"{counter}: missing copy ({len(copy_k)}) or slim ({len(slim_k)}) dispatches")
        copy_kib = statistics.median(sorted(copy_k)[-3:])     # the three calibration copies
        scale = (COPY_CALIB_BYTES / 1024.0) / copy_kib
        n = min(len(v) for v in slim_k.values())
        calls = n if calls is None else min(calls, n)
        per_call_kib = sum(statistics.mean(v) for v in slim_k.values())
        out[f"{key}_kib_raw_per_call"] = round(per_call_kib, 1)
        out[f"{key}_kernels_kib_raw"] = {k: round(statistics.mean(v), 1) for k, v in slim_k.items()}
        out[f"copy_{key}_kib_raw"] = round(copy_kib, 1)
        out[f"{key}_scale"] = round(scale, 4)
        out[f"{key}_bytes_per_call"] = int(per_call_kib * 1024 * scale)
    out["calls"] = calls
    out["hbm_bytes_per_call"] = out["fetch_bytes_per_call"] + out["write_bytes_per_call"]
    out["algorithmic_bytes_per_call"] = alg_bytes(*HEADLINE)
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def profile_run(torch, slim, shape, calls=30, qa=False):
    """A short run for rocprofv3: `calls` slim_linear calls (slim_linear_qa
    with qa=True) of one shape (the headline by default) on a pool of buffer
    sets, then COPY_CALIB_BYTES copied three times by torch (the byte
    counters' calibration)."""
    M, N, K, r = shape
    pool = (QALayerPool if qa else LayerPool)(torch, slim, M, N, K, r, 256 << 20)
    for i in range(calls):
        pool.call(slim, i)
    torch.cuda.synchronize()
    a = torch.empty(COPY_CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"profile run done: {calls} slim_linear{'_qa' if qa else ''} calls at M={M} N={N} K={K} r={r}, "
          f"3 copies of {COPY_CALIB_BYTES >> 20} MiB", flush=True)


def sweep(torch, slim, r, steps):
    """Decoder-block sweep: slim_linear and a dense fp16 matmul per shape."""
    res = {}
    for (name, N, K) in SWEEP_SHAPES:
        for M in SWEEP_M:
            t = statistics.median(bench_slim(torch, slim, M, N, K, r, steps, 5, reps=3))
            td = bench_dense(torch, M, N, K, steps, 5)
            us, usd = t * 1e3, td * 1e3
            b, fl = alg_bytes(M, N, K, r), alg_flops(M, N, K, r)
            res[f"{name}@M{M}"] = {
                "M": M, "N": N, "K": K, "us_per_call": round(us, 3), "GB/s": round(b / us / 1e3, 1),
                "TFLOP/s": round(fl / us / 1e6, 2), "roofline_frac": round(t_roof_us(M, N, K, r) / us, 4),
                "bound": "hbm" if alg_bytes(M, N, K, r) / HBM_PEAK_GBS / 1e3 >= fl / FP16_PEAK_TFLOPS / 1e6
                else "mfma",
                "dense_fp16_us": round(usd, 3), "speedup_vs_dense": round(usd / us, 3)}
            log(f"sweep {name}@M{M}: {us:.2f} us (dense {usd:.2f} us)")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true", help="short headline run + copy, for rocprofv3")
    ap.add_argument("--shape", nargs=4, type=int, metavar=("M", "N", "K", "R"), default=list(HEADLINE),
                    help="shape of the --profile run")
    ap.add_argument("--qa", action="store_true", help="with --profile: quantised adapters (slim_linear_qa)")
    ap.add_argument("--transposed", action="store_true",
                    help="with --profile: slim_pack_transposed of the N x K weight of --shape, 30 calls")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this build has no "
              f"multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    slim._lib.load()
    if args.profile and args.transposed:
        _, N, K, _ = args.shape
        t = bench_pack_transposed(torch, slim, N, K, 30, 3) * 1e3
        log(f"pack_transposed {N}x{K}: {t:.2f} us/call, {N * K * (25 / 64 + 9 / 8) / t / 1e3:.0f} GB/s")
        return
    if args.profile:
        profile_run(torch, slim, tuple(args.shape), qa=args.qa)
        return

    M, N, K, r = HEADLINE
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
    }
    traffic, tnote = traffic_from_profile(M, N, K, r, nbytes)
    out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                       "per_launch_bytes": nbytes, "traffic_note": tnote,
                       "note": "one slim_linear call is the timed unit: at this shape ONE launch "
                               "(decode_twave_kernel: rows of T, main term and T.R); "
                               "achieved = algorithmic bytes per call / us per call"}
    if not args.quick:
        extra = {}
        sw = sweep(torch, slim, r, max(20, args.steps // 4))
        extra["sweep"] = sw
        down = sw["down@M2048"]
        extra["down_M2048"] = {"us_per_call": down["us_per_call"], "TFLOP/s": down["TFLOP/s"],
                               "mfma_frac": round(down["TFLOP/s"] / FP16_PEAK_TFLOPS, 4)}
        extra["speedup_vs_dense_M1"] = sw["qkvo@M1"]["speedup_vs_dense"]
        extra["quantized_adapters"] = bench_qa(torch, slim, r, max(20, args.steps // 4), sw)
        extra["input_8bit"] = bench_a8(torch, slim, r, max(20, args.steps // 4), sw)
        extra["hybrid_tiles"] = bench_hybrid(torch, slim, r, max(20, args.steps // 4), sw)
        tpk = bench_pack(torch, slim, 4096, 4096, 50, 5)
        extra["pack_q_proj"] = {"us_per_call": round(tpk * 1e3, 2),
                                "GB/s": round(4096 * 4096 * (4 + 25 / 64) / (tpk * 1e-3) / 1e9, 1)}
        tpt = bench_pack_transposed(torch, slim, 4096, 4096, 50, 5)
        extra["pack_transposed_q_proj"] = {"us_per_call": round(tpt * 1e3, 2),
                                           "GB/s": round(4096 * 4096 * (25 / 64 + 9 / 8) / (tpt * 1e-3) / 1e9, 1)}
        extra["gpu_clock"] = gpu_clock()
        out["extra"] = extra
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
