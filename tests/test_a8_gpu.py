"""The layer with an 8-bit input (slim_quantize_input, slim_linear_a8) on the
GPU against the fp64 oracle.

slim_quantize_input must match oracle.quantize_input byte for byte.  The
layer takes the oracle's own codes and scales as input (copied to the GPU),
so nothing the GPU computed enters the reference; it must meet the linear
layer's bars (relative Frobenius error <= 2e-3, max|err| <= 1e-2 max|y_ref|)
against oracle.linear_a8.  Prefill shapes run the int8 sparse matrix core,
decode shapes the fp16 kernels on the dequantised input."""
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


def _quant_on_gpu(env, X):
    torch, slim = env
    q, s = slim.quantize_input(to_dev(X, torch))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("case", [wl.QPROJ, wl.QPROJ.with_M(16), wl.GATEUP, wl.DOWN, wl.TINY],
                         ids=lambda c: f"{c.name}@M{c.M}")
def test_quantize_input_bit_exact(env, case):
    X = wl.make_inputs(case).X
    print(f"[a8 quant] {case.name} M={X.shape[0]} K={X.shape[1]}", flush=True)
    q, s = _quant_on_gpu(env, X)
    qo, so = oracle.quantize_input(X)
    assert np.array_equal(q, qo)
    assert np.array_equal(s.view(np.uint16), so.view(np.uint16))


def test_quantize_input_edge_rows(env):
    rng = np.random.default_rng(50)
    X = wl.random_fp16(rng, (12, 1024))
    X[0] = 0                                             # zero row: s = 0, q = 0
    X[1] = np.float16(-0.0)
    X[2, :] = np.float16(0.5); X[2, 7] = np.float16(127.0)       # x / s lands on exact halves
    X[3] *= np.float16(1e-3)                             # subnormal-range scale
    X[4, 100] = np.float16(65504.0)                      # the largest fp16
    X[5, :] = np.float16(-3.0)                           # constant row: all +-127
    X[6, ::2] = np.float16(2.5); X[6, 1] = np.float16(127.0)
    X[7] *= np.float16(300)                              # large values
    X[8, 5] = np.float16(-6e-8)                          # a subnormal input element
    q, s = _quant_on_gpu(env, X)
    qo, so = oracle.quantize_input(X)
    assert np.array_equal(q, qo)
    assert np.array_equal(s.view(np.uint16), so.view(np.uint16))
    # rows longer than the quantiser keeps in registers (read twice), and short ones
    for K in (20480, 8, 2056):
        Xl = wl.random_fp16(rng, (3, K))
        Xl[1, K // 2] = np.float16(-700.0)
        q, s = _quant_on_gpu(env, Xl)
        qo, so = oracle.quantize_input(Xl)
        assert np.array_equal(q, qo), K
        assert np.array_equal(s.view(np.uint16), so.view(np.uint16)), K


def _run(env, case, sample_rows=None, no_adapter=False):
    torch, slim = env
    print(f"[a8 linear] {case.name} M={case.M} N={case.N} K={case.K} r={case.r} rows={sample_rows is not None}",
          flush=True)
    inp = wl.make_inputs(case)
    (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
    qx, sx = oracle.quantize_input(inp.X)
    L, R = (None, None) if no_adapter else (inp.L, inp.R)
    dL = None if L is None else to_dev(L.T, torch)
    dR = None if R is None else to_dev(R.T, torch)
    Y = slim.linear_a8(to_dev(qx, torch), to_dev(sx, torch), w, dL, dR)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    ref = oracle.linear_a8(qx, sx, v, m, s, L, R, rows=sample_rows)
    if sample_rows is not None:
        Y = Y[sample_rows]
    return assert_close_to_oracle(Y, ref, case.name)


def _rows(M, seed):
    rng = np.random.default_rng(seed)
    rows = [b + int(rng.integers(0, min(128, M - b))) for b in range(0, M, 128)]
    return np.unique(np.asarray(rows + [0, M - 1], dtype=np.int64))


@pytest.mark.parametrize("case", [wl.QPROJ, wl.QPROJ.with_M(16), wl.GATEUP, wl.TINY,
                                  wl.Case("gate_proj@M256", M=256, N=11008, K=4096, r=416)],
                         ids=lambda c: f"{c.name}@M{c.M}")
def test_linear_a8_dequantised_input_path(env, case):
    _run(env, case)


def test_linear_a8_down_prefill(env):
    """down at 2048 tokens with the adapter: the dequantised input on the
    one-pass fp16 prefill."""
    _run(env, wl.DOWN, sample_rows=_rows(wl.DOWN.M, 5))


def test_linear_a8_int8_core_no_adapter(env):
    """The int8 core (prefill shapes without an adapter): down at 2048
    tokens, and partial last token and row tiles (272 tiles)."""
    _run(env, wl.DOWN, sample_rows=_rows(wl.DOWN.M, 8), no_adapter=True)
    _run(env, wl.Case("a8_ragged_r0", M=2000, N=4112, K=1024, r=64, seed=93), sample_rows=_rows(2000, 9),
         no_adapter=True)


@pytest.mark.parametrize("name,N,K", [("q_proj", 4096, 4096), ("gate_proj", 11008, 4096)])
def test_linear_a8_prefill_sweep(env, name, N, K):
    case = wl.Case(f"{name}@M2048", M=2048, N=N, K=K, r=wl.RANK)
    _run(env, case, sample_rows=_rows(2048, 6))


def test_linear_a8_prefill_ragged_and_no_adapter(env):
    """Partial last token and row tiles (272 tiles) with an adapter, and the
    int8 core without one."""
    case = wl.Case("a8_ragged", M=2000, N=4112, K=1024, r=64, seed=91)
    _run(env, case, sample_rows=_rows(2000, 7))
    _run(env, wl.Case("a8_r0", M=1024, N=4096, K=2048, r=32, seed=92), no_adapter=True)
