"""Seeded random shapes through every dispatch path (one-launch decode with
one or three row blocks, two-launch decode, K-split decode with 4/6/8-block
row groups, prefill with and without a K split, generic), with fp16 and with
quantised adapters, against the fp64 oracle at the linear layer's bars."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close_to_oracle, pack_on_gpu, to_dev

pytestmark = pytest.mark.gpu


def _shapes(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 64, 130, 260]))
        N = 16 * int(rng.integers(1, 751))
        K = 128 * int(rng.integers(1, 49))
        r = 32 * int(rng.integers(0, 17))
        if M * N * K > 1_500_000_000:          # keep the oracle to about a second
            continue
        out.append((M, N, K, r, int(rng.integers(1 << 30))))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module")
def env():
    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    slim._lib.load()
    return torch, slim


@pytest.mark.parametrize("M,N,K,r,seed", SHAPES, ids=[f"M{s[0]}-N{s[1]}-K{s[2]}-r{s[3]}" for s in SHAPES])
def test_random_shape(env, M, N, K, r, seed):
    torch, slim = env
    print(f"[random] M={M} N={N} K={K} r={r} seed={seed}", flush=True)
    inp = wl.make_inputs(wl.Case("random", M=M, N=N, K=K, r=r, seed=seed))
    (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
    dX = to_dev(inp.X, torch)
    if r == 0:
        Y = slim.linear(dX, w, None, None).cpu().numpy()
        assert_close_to_oracle(Y, oracle.linear(inp.X, v, m, s, None, None), "r=0")
        return
    Y = slim.linear(dX, w, to_dev(inp.L.T, torch), to_dev(inp.R.T, torch)).cpu().numpy()
    assert_close_to_oracle(Y, oracle.linear(inp.X, v, m, s, inp.L, inp.R), "fp16 adapters")
    qa = slim.pack_adapters(to_dev(np.asarray(inp.L, np.float32).T, torch), to_dev(np.asarray(inp.R, np.float32).T, torch))
    Yq = slim.linear_qa(dX, w, qa).cpu().numpy()
    lq = qa.lq.cpu().numpy().reshape(r, K // 2)
    ls = qa.ls.cpu().numpy().view(np.float16).reshape(r, K // 128)
    rq = qa.rq.cpu().numpy().reshape(N, r // 2)
    rs = qa.rs.cpu().numpy().view(np.float16).reshape(N, r // 32)
    assert_close_to_oracle(Yq, oracle.linear_qa(inp.X, v, m, s, lq, ls, rq, rs, r), "quantised adapters")
