"""The one-pass prefill path (T = X.L first, then one kernel that runs the 2:4
sparse chunks of X.deq(W_c)^T and the dense chunks of T.R into the same
accumulators) against the fp64 oracle, on shapes that reach it (more than
128 tiles of 256 rows x 128 tokens):

  - no adapter (r = 0: no T, no dense chunks);
  - r = 32: one half-filled dense chunk, and ragged N (17 row tiles) with M
    not a multiple of 128;
  - r = 608: three T column tiles and a partial dense chunk;
  - T without a K split (at least 256 T tiles);
  - 129 tiles (the fewest this path takes: three ragged token tiles) and a
    16-way K split of T;
  - slim_linear_batched (grid over problems, per-problem workspace);
  - quantised adapters at prefill (dequantised into the workspace, then this
    path).

Rows of Y are independent: large cases check sampled token rows, at least one
in every 128-token tile."""
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


def _rows(M, seed):
    rng = np.random.default_rng(seed)
    rows = [b + int(rng.integers(0, min(128, M - b))) for b in range(0, M, 128)]
    return np.unique(np.asarray(rows + [0, M - 1], dtype=np.int64))


def _run(env, case, sample=True):
    torch, slim = env
    print(f"[kx] {case.name} M={case.M} N={case.N} K={case.K} r={case.r}", flush=True)
    inp = wl.make_inputs(case)
    (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
    L, R = (inp.L, inp.R) if case.r > 0 else (None, None)
    Y = slim.linear(to_dev(inp.X, torch), w, None if L is None else to_dev(L.T, torch),
                    None if R is None else to_dev(R.T, torch))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    rows = _rows(case.M, case.seed + 17) if sample else None
    ref = oracle.linear(inp.X, v, m, s, L, R, rows=rows)
    if rows is not None:
        Y = Y[rows]
    return assert_close_to_oracle(Y, ref, case.name)


@pytest.mark.parametrize("case", [
    wl.Case("kx_r0", M=2048, N=4096, K=1024, r=0, seed=31),
    wl.Case("kx_r32_ragged", M=1500, N=4352, K=1152, r=32, seed=32),
    wl.Case("kx_r608", M=2048, N=4096, K=512, r=608, seed=33),
    wl.Case("kx_t_unsplit", M=16512, N=512, K=256, r=32, seed=34),
    wl.Case("kx_129_tiles", M=380, N=11008, K=1024, r=416, seed=36),
], ids=lambda c: c.name)
def test_prefill_kx_shapes(env, case):
    _run(env, case)


def test_prefill_kx_batched(env):
    torch, slim = env
    B, M, N, K, r = 2, 1024, 6144, 512, 64          # 24 x 8 = 192 tiles per problem
    cases = [wl.Case("kxb", M=M, N=N, K=K, r=r, seed=200 + b) for b in range(B)]
    inps = [wl.make_inputs(c) for c in cases]
    packs = [pack_on_gpu(i.W, torch, slim) for i in inps]
    X = np.stack([i.X for i in inps])
    dX = to_dev(X, torch)
    dV = torch.stack([p[1].values for p in packs]).contiguous()
    dM = torch.stack([p[1].meta for p in packs]).contiguous()
    dS = torch.stack([p[1].scales for p in packs]).contiguous()
    dL = to_dev(np.stack([i.L.T for i in inps]), torch)
    dR = to_dev(np.stack([i.R.T for i in inps]), torch)
    dY = torch.empty((B, M, N), dtype=torch.float16, device="cuda")
    ws = slim.workspace(M, N, K, r, batch=B)
    print(f"[kx batched] B={B} M={M} N={N} K={K} r={r}", flush=True)
    slim.slim_linear_batched(B, M, N, K, r, dX, M * K, dV, N * K // 4, dM, N * K // 8, dS, N * K // 128,
                             dL, K * r, dR, r * N, dY, M * N, ws)
    torch.cuda.synchronize()
    Y = dY.cpu().numpy()
    for b in range(B):
        v, m, s = packs[b][0]
        rows = _rows(M, 50 + b)
        ref = oracle.linear(X[b], v, m, s, inps[b].L, inps[b].R, rows=rows)
        assert_close_to_oracle(Y[b][rows], ref, f"kx batched[{b}]")


def test_prefill_kx_quantised_adapters(env):
    torch, slim = env
    case = wl.Case("kx_qa", M=2048, N=4096, K=1024, r=128, seed=35)
    print(f"[kx qa] M={case.M} N={case.N} K={case.K} r={case.r}", flush=True)
    inp = wl.make_inputs(case)
    (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
    qa = slim.pack_adapters(to_dev(inp.L.T, torch).float(), to_dev(inp.R.T, torch).float())
    Y = slim.linear_qa(to_dev(inp.X, torch), w, qa)
    torch.cuda.synchronize()
    lq, ls, rq, rs = oracle.pack_adapters(inp.L, inp.R)
    rows = _rows(case.M, 60)
    ref = oracle.linear_qa(inp.X, v, m, s, lq, ls, rq, rs, case.r, rows=rows)
    assert_close_to_oracle(Y.cpu().numpy()[rows], ref, "kx qa")
