"""Quantised adapters on the GPU against the fp64 CPU oracle.

slim_pack_adapter must match the oracle's adapter quantiser bit for bit;
slim_linear_qa must meet the linear layer's bar (relative Frobenius error
<= 2e-3, max|err| <= 1e-2 * max|y_ref|) against Y computed from the same
packed weight and the same packed adapter factors, on every path it takes:
the kernels that read the int4 factors (one or two tokens in one launch or
in two, 3 to 16 tokens on the K-split path) and the dequantise-then-fp16
path (every other shape)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close_to_oracle, pack_on_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    slim._lib.load()
    return torch, slim


def _pack_adapters_gpu(env, L, R):
    torch, slim = env
    Lt = to_dev(np.asarray(L, dtype=np.float32).T, torch)
    Rt = to_dev(np.asarray(R, dtype=np.float32).T, torch)
    qa = slim.pack_adapters(Lt, Rt)
    torch.cuda.synchronize()
    return qa


def _host(qa):
    r, K, N = qa.r, qa.K, qa.N
    return (qa.lq.cpu().numpy().reshape(r, K // 2), qa.ls.cpu().numpy().view(np.float16).reshape(r, K // 128),
            qa.rq.cpu().numpy().reshape(N, r // 2), qa.rs.cpu().numpy().view(np.float16).reshape(N, r // 32))


def _assert_pack_equal(got, ref, what):
    for name, g, e in zip(("lq", "ls", "rq", "rs"), got, ref):
        assert g.shape == e.shape, (what, name, g.shape, e.shape)
        if g.dtype == np.float16:
            g, e = g.view(np.uint16), np.asarray(e, dtype=np.float16).view(np.uint16)
        bad = np.argwhere(g != e)
        assert bad.size == 0, f"{what}: {name} differs at {bad[:5].tolist()} ({bad.shape[0]} entries)"


@pytest.mark.parametrize("K,N,r", [(4096, 4096, 416), (512, 512, 32), (11008, 4096, 416), (128, 16, 64)])
def test_pack_adapter_bit_exact(env, K, N, r):
    print(f"[qa-pack] K={K} N={N} r={r}", flush=True)
    inp = wl.make_inputs(wl.Case("qa", M=1, N=N, K=K, r=r, seed=K + N + r))
    got = _host(_pack_adapters_gpu(env, inp.L, inp.R))
    _assert_pack_equal(got, oracle.pack_adapters(inp.L, inp.R), f"K={K} N={N} r={r}")


def test_pack_adapter_edge_values(env):
    """Zero groups (scale 0, codes 0), exact half-way ratios (ties to even),
    a single large entry per group, negative maxima and fp32 inputs far
    outside the fp16 range of the adapters."""
    rng = np.random.default_rng(7)
    K, N, r = 256, 64, 64
    L = rng.standard_normal((K, r)).astype(np.float32) * np.float32(0.05)
    R = rng.standard_normal((r, N)).astype(np.float32) * np.float32(0.05)
    L[:128, 0] = 0.0                                   # one zero group of Lt row 0
    L[:, 1] = 0.0                                      # Lt row 1 all zero
    L[:128, 2] = np.float32(0.5) * (np.arange(128) % 15 - 7)   # 7 * 0.5 -> s = 0.5 exactly ...
    L[5, 2] = np.float32(0.75)                         # ... so 0.75 / 0.5 = 1.5 rounds to 2
    L[6, 2] = np.float32(1.25)                         # 2.5 rounds to 2
    L[7, 2] = np.float32(-1.75)                        # -3.5 rounds to -4
    L[128:, 3] = 0.0
    L[200, 3] = np.float32(-3.0)                       # negative maximum: code -7
    R[:32, 0] = 0.0                                    # zero group of Rt row 0
    R[:, 1] *= np.float32(1e4)                         # large values
    R[32:, 2] = np.float32(1e-6) * rng.standard_normal(32).astype(np.float32)   # tiny scale
    got = _host(_pack_adapters_gpu(env, L, R))
    ref = oracle.pack_adapters(L, R)
    _assert_pack_equal(got, ref, "edge values")
    q = oracle.unpack_adapter(got[0], K)
    assert np.all(q[1] == 0) and np.all(got[1][1].astype(np.float32) == 0)
    assert q[2, 5] == 2 and q[2, 6] == 2 and q[2, 7] == -4
    assert q[3, 200] == -7


def _qa_case(env, X, W, L, R, what, sample_rows=None, ws=None):
    torch, slim = env
    M, K = X.shape
    N = W.shape[0]
    r = L.shape[1]
    print(f"[qa-linear] {what} M={M} N={N} K={K} r={r}", flush=True)
    (v, m, s), w = pack_on_gpu(W, torch, slim)
    qa = _pack_adapters_gpu(env, L, R)
    lq, ls, rq, rs = _host(qa)
    Y = slim.linear_qa(to_dev(X, torch), w, qa, ws=ws)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    Y_ref = oracle.linear_qa(X, v, m, s, lq, ls, rq, rs, r, rows=sample_rows)
    if sample_rows is not None:
        Y = Y[sample_rows]
    return assert_close_to_oracle(Y, Y_ref, what)


@pytest.mark.parametrize("case", [wl.QPROJ, wl.QPROJ.with_M(2), wl.DOWN.with_M(1), wl.DOWN.with_M(2),
                                  wl.GATEUP.with_M(1), wl.GATEUP.with_M(2), wl.QPROJ.with_M(3),
                                  wl.QPROJ.with_M(16), wl.GATEUP, wl.DOWN.with_M(16), wl.TINY],
                         ids=lambda c: f"{c.name}@M{c.M}")
def test_linear_qa_workloads(env, case):
    inp = wl.make_inputs(case)
    _qa_case(env, inp.X, inp.W, inp.L, inp.R, f"{case.name}@M{case.M}")


def test_linear_qa_prefill_sampled(env):
    case = wl.DOWN
    inp = wl.make_inputs(case)
    rows = np.sort(np.concatenate([np.random.default_rng(3).choice(case.M, 40, replace=False), [0, case.M - 1]]))
    _qa_case(env, inp.X, inp.W, inp.L, inp.R, "down@M2048 (sampled rows)", sample_rows=rows)


@pytest.mark.parametrize("N,K,r,M", [(16, 128, 32, 1), (128, 256, 32, 1), (1040, 1152, 96, 1), (1040, 1152, 96, 2),
                                     (272, 11008, 416, 1), (1024, 1024, 64, 3), (1040, 1152, 96, 5),
                                     (2048, 1152, 256, 9), (16, 128, 32, 8), (1024, 1024, 64, 257),
                                     (11008, 128, 32, 17), (11200, 1024, 256, 1), (8192, 2048, 192, 2),
                                     (11200, 1024, 256, 9), (4000, 11008, 416, 7)])
def test_linear_qa_shapes(env, N, K, r, M):
    inp = wl.make_inputs(wl.Case("qa-shape", M=M, N=N, K=K, r=r, seed=N + K + r + M))
    _qa_case(env, inp.X, inp.W, inp.L, inp.R, f"N={N} K={K} r={r} M={M}")


def test_linear_qa_zero_and_large_adapters(env):
    case = wl.Case("qz", M=1, N=4096, K=4096, r=416, seed=11)
    inp = wl.make_inputs(case)
    _qa_case(env, inp.X, inp.W, np.zeros_like(inp.L), inp.R, "L = 0")
    _qa_case(env, inp.X, np.zeros_like(inp.W), inp.L * np.float16(8), inp.R, "W = 0, adapter only")


def test_linear_qa_workspace_shared_with_fp16_calls(env):
    """One workspace serves fp16-adapter and quantised-adapter calls of
    several shapes in turn; every result equals that of a fresh workspace."""
    torch, slim = env
    cases = [wl.QPROJ, wl.QPROJ.with_M(16), wl.DOWN.with_M(1), wl.QPROJ.with_M(2), wl.GATEUP.with_M(1), wl.GATEUP]
    big = max(max(slim.slim_linear_qa_workspace_bytes(c.M, c.N, c.K, c.r),
                  slim.slim_linear_workspace_bytes(c.M, c.N, c.K, c.r)) for c in cases)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    prepared = []
    for c in cases:
        inp = wl.make_inputs(c)
        _, w = pack_on_gpu(inp.W, torch, slim)
        qa = _pack_adapters_gpu(env, inp.L, inp.R)
        dX, dL, dR = to_dev(inp.X, torch), to_dev(inp.L.T, torch), to_dev(inp.R.T, torch)
        prepared.append((c, w, qa, dX, dL, dR,
                         slim.linear_qa(dX, w, qa).cpu().numpy(), slim.linear(dX, w, dL, dR).cpu().numpy()))
    for rep in range(2):
        for c, w, qa, dX, dL, dR, y_qa, y_fp in prepared:
            print(f"[qa-ws] rep={rep} {c.name}@M{c.M}", flush=True)
            assert np.array_equal(slim.linear_qa(dX, w, qa, ws=ws).cpu().numpy(), y_qa)
            assert np.array_equal(slim.linear(dX, w, dL, dR, ws=ws).cpu().numpy(), y_fp)


def test_linear_qa_in_captured_graph_replays(env):
    torch, slim = env
    for case in (wl.QPROJ, wl.QPROJ.with_M(16), wl.GATEUP.with_M(1), wl.GATEUP):
        print(f"[qa-graph] {case.name}@M{case.M}", flush=True)
        inp = wl.make_inputs(case)
        _, w = pack_on_gpu(inp.W, torch, slim)
        qa = _pack_adapters_gpu(env, inp.L, inp.R)
        dX = to_dev(inp.X, torch)
        ws = slim.workspace_qa(case.M, case.N, case.K, case.r)
        Y_eager = slim.linear_qa(dX, w, qa, ws=ws).clone()
        Y = torch.zeros_like(Y_eager)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                slim.linear_qa(dX, w, qa, ws=ws, out=Y)
        torch.cuda.current_stream().wait_stream(cap)
        for rep in range(3):
            Y.zero_()
            slim.linear_qa(dX, w, qa, ws=ws)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Y_eager), f"replay {rep}"
