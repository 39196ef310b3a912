"""slim_linear_noalloc (the library's own per-GPU scratch, no workspace
argument) against slim_linear with a caller workspace: the same kernels run,
so the outputs are bit-identical, and both meet the oracle's bar.  Calls in a
row reuse the one scratch array, each later one with a smaller input than the
one before (the K-split decode at 16 tokens, the one-launch decode at one
token whose hand-off state lives in that array, the tiny configuration)."""
import ctypes

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


def _call_noalloc(slim, torch, dX, w, dL, dR):
    Y = torch.empty((dX.shape[0], w.N), dtype=torch.float16, device="cuda")
    lib = slim._lib.load()
    st = lib.slim_linear_noalloc(ctypes.c_void_p(dX.data_ptr()), dX.shape[0], w.N, w.K,
                                 ctypes.c_void_p(w.values.data_ptr()), ctypes.c_void_p(w.meta.data_ptr()),
                                 ctypes.c_void_p(w.scales.data_ptr()), 128, ctypes.c_void_p(dL.data_ptr()),
                                 ctypes.c_void_p(dR.data_ptr()), dL.shape[0], ctypes.c_void_p(Y.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.slim_last_error().decode()
    return Y


def test_noalloc_matches_slim_linear_on_calls_in_a_row(env):
    torch, slim = env
    for case in (wl.QPROJ.with_M(16), wl.QPROJ, wl.TINY, wl.QPROJ):
        print(f"[noalloc] {case.name} M={case.M} N={case.N} K={case.K} r={case.r}", flush=True)
        inp = wl.make_inputs(case)
        (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
        dX, dL, dR = to_dev(inp.X, torch), to_dev(inp.L.T, torch), to_dev(inp.R.T, torch)
        Y_na = _call_noalloc(slim, torch, dX, w, dL, dR)
        Y_ws = slim.linear(dX, w, dL, dR)
        torch.cuda.synchronize()
        assert torch.equal(Y_na, Y_ws), f"{case.name}: slim_linear_noalloc differs from slim_linear"
        assert_close_to_oracle(Y_na.cpu().numpy(), oracle.linear(inp.X, v, m, s, inp.L, inp.R), case.name)


def test_noalloc_rejects_shapes_beyond_its_scratch(env):
    torch, slim = env
    lib = slim._lib.load()
    M, N, K, r = 100000, 16, 128, 4096
    assert slim.slim_linear_workspace_bytes(M, N, K, r) > 64 << 20
    p = ctypes.c_void_p(256)
    st = lib.slim_linear_noalloc(p, M, N, K, p, p, p, 128, p, p, r, p, None)
    assert st == 1 and b"maximum" in lib.slim_last_error()
    assert np.isfinite(1.0)
