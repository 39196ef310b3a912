"""Hybrid dense / 2:4 tiles (slim_pack_hybrid, slim_linear_hybrid) on the GPU
against the fp64 oracle.

The pack must match oracle.pack_hybrid byte for byte.  The layer takes the
oracle's own packed arrays as input (copied to the GPU), so no GPU-made
operand enters the reference, and must meet the linear layer's bars against
oracle.linear_hybrid on the two-launch decode kernel (1-16 tokens), the
prefill kernel with and without a K split, and the generic kernel."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import assert_close_to_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    slim._lib.load()
    return torch, slim


def _flags(N, K, p, seed):
    rng = np.random.default_rng(seed)
    return (rng.random(((N + 15) // 16, K // 128)) < p).astype(np.int32)


@pytest.mark.parametrize("N,K,p", [(4096, 4096, 0.25), (4096, 4096, 0.0), (4096, 4096, 1.0), (37, 640, 0.5),
                                   (11008, 4096, 0.5)])
def test_pack_hybrid_bit_exact(env, N, K, p):
    torch, slim = env
    print(f"[hybrid pack] N={N} K={K} dense={p}", flush=True)
    rng = np.random.default_rng(N + K)
    W = wl.random_weights(rng, N, K)
    flags = _flags(N, K, p, N)
    w = slim.pack_hybrid(to_dev(W, torch), to_dev(flags, torch))
    torch.cuda.synchronize()
    v, m, s, d = oracle.pack_hybrid(W, flags)
    assert np.array_equal(w.values.cpu().numpy(), v)
    assert np.array_equal(w.meta.cpu().numpy(), m)
    assert np.array_equal(w.scales.cpu().numpy().view(np.uint16), s.view(np.uint16))
    assert np.array_equal(w.dvalues.cpu().numpy(), d)


def _run(env, case, p, sample_rows=None, no_adapter=False):
    torch, slim = env
    print(f"[hybrid linear] {case.name} M={case.M} N={case.N} K={case.K} r={case.r} dense={p}", flush=True)
    inp = wl.make_inputs(case)
    flags = _flags(case.N, case.K, p, case.seed + 7)
    v, m, s, d = oracle.pack_hybrid(inp.W, flags)
    w = slim.HybridWeight(to_dev(v, torch), to_dev(m, torch), to_dev(s, torch), to_dev(d, torch),
                          to_dev(flags, torch), case.N, case.K)
    L, R = (None, None) if no_adapter else (inp.L, inp.R)
    Y = slim.linear_hybrid(to_dev(inp.X, torch), w, None if L is None else to_dev(L.T, torch),
                           None if R is None else to_dev(R.T, torch))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    ref = oracle.linear_hybrid(inp.X, v, m, s, d, L, R, rows=sample_rows)
    if sample_rows is not None:
        Y = Y[sample_rows]
    return assert_close_to_oracle(Y, ref, f"{case.name} dense={p}")


@pytest.mark.parametrize("M", [1, 2, 3, 16])
@pytest.mark.parametrize("p", [0.0, 0.5, 1.0])
def test_linear_hybrid_decode(env, M, p):
    _run(env, wl.QPROJ.with_M(M), p)


def test_linear_hybrid_decode_gate_up_and_no_adapter(env):
    _run(env, wl.GATEUP, 0.3)
    _run(env, wl.Case("hyb_r0", M=4, N=1024, K=1152, r=32, seed=3), 0.5, no_adapter=True)


def test_linear_hybrid_prefill(env):
    rows = np.unique(np.concatenate([np.arange(0, 2048, 128) + 5, [0, 2047]]))
    _run(env, wl.DOWN, 0.5, sample_rows=rows)
    _run(env, wl.Case("hyb_q2048", M=2048, N=4096, K=4096, r=416), 0.25, sample_rows=rows)


def test_linear_hybrid_prefill_k_split_and_ragged(env):
    _run(env, wl.Case("hyb_q256", M=256, N=4096, K=4096, r=416), 0.5)          # K split over 8
    _run(env, wl.Case("hyb_ragged", M=300, N=4112, K=1024, r=64, seed=11), 0.5)


def test_linear_hybrid_generic_fallback(env):
    """r/32 adapter column blocks above the 256-row tiles: the generic kernel."""
    _run(env, wl.Case("hyb_generic", M=20, N=48, K=256, r=64, seed=12), 0.5)
