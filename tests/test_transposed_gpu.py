"""Double-pruned transpose (SLoPe's backward operand) on the GPU against the
CPU oracle: slim_pack_transposed must match oracle.pack_transposed bit for
bit, values and metadata, on packed weights made by slim_pack."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import pack_on_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    slim._lib.load()
    return torch, slim


def _check(env, W, what):
    torch, slim = env
    N, K = W.shape
    print(f"[transposed] {what} N={N} K={K}", flush=True)
    (v, m, s), w = pack_on_gpu(W, torch, slim)
    tv, tm = slim.pack_transposed(w)
    torch.cuda.synchronize()
    got_v = tv.cpu().numpy().view(np.uint16)
    got_m = tm.cpu().numpy().view(np.uint16)
    ref_v, ref_m = oracle.pack_transposed(v, m, s, N, K)
    assert got_v.shape == ref_v.shape and got_m.shape == ref_m.shape
    bad = np.argwhere(got_v != ref_v.view(np.uint16))
    assert bad.size == 0, f"{what}: tvalues differ at {bad[:5].tolist()} ({bad.shape[0]} entries)"
    bad = np.argwhere(got_m != ref_m)
    assert bad.size == 0, f"{what}: tmeta differs at {bad[:5].tolist()} ({bad.shape[0]} entries)"


@pytest.mark.parametrize("N,K", [(16, 128), (128, 256), (144, 384), (4096, 4096), (11008, 4096), (4096, 11008),
                                 (1040, 1152), (272, 128), (2064, 640), (16, 28672), (8192, 128), (48, 16384)])
def test_pack_transposed_bit_exact(env, N, K):
    """Full workload weights, a single row block, row-block counts that are
    not multiples of the 8 a workgroup takes, several k groups, one row block
    with a very long K (224 groups), and one k group with a very wide N."""
    rng = np.random.default_rng(N * 7 + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    _check(env, W, "gaussian")


def test_pack_transposed_ties_and_zeros(env):
    """Small-integer weights (many equal magnitudes along n, so the
    lower-index rule decides), all-zero groups and rows, a transposable
    mask that must come back unpruned, and extreme fp16 scales."""
    torch, slim = env
    rng = np.random.default_rng(17)
    N, K = 160, 512
    W = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    W[:, ::128] = 7
    W[:16, 128:256] = 0.0                      # one zero group of a whole row block
    W[40] = 0.0                                # a zero row
    W[64:80] *= np.float32(6e4 / 7)            # scales near the fp16 maximum
    W[96:112] *= np.float32(1e-6)              # subnormal fp16 scales
    _check(env, W, "ties")
    mask = np.zeros((4, 4), dtype=bool)
    mask[:2, :2] = mask[2:, 2:] = True
    Wt = (rng.standard_normal((N, K)) * np.tile(mask, (N // 4, K // 4))).astype(np.float32)
    _check(env, Wt, "transposable")
    (v, m, s), w = pack_on_gpu(Wt, torch, slim)
    tv, tm = slim.pack_transposed(w)
    D = oracle.dequantize(oracle.unpack(v, m, K), s).astype(np.float16)
    assert np.array_equal(oracle.unpack_transposed(tv.cpu().numpy(), tm.cpu().numpy().view(np.uint16), N), D.T)


def test_pack_transposed_workloads(env):
    for case in (wl.QPROJ, wl.DOWN):
        inp = wl.make_inputs(case.with_M(1))
        _check(env, inp.W, case.name)


def test_pack_transposed_in_captured_graph_replays(env):
    """Captured once, replayed three times with eager calls on other
    weights in between: every replay rewrites the same bytes."""
    torch, slim = env
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((1040, 1152)) * 0.02).astype(np.float32)
    Wo = (rng.standard_normal((4096, 4096)) * 0.02).astype(np.float32)
    _, w = pack_on_gpu(W, torch, slim)
    _, wo = pack_on_gpu(Wo, torch, slim)
    ref_v, ref_m = slim.pack_transposed(w)
    tv, tm = torch.zeros_like(ref_v), torch.zeros_like(ref_m)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            slim.slim_pack_transposed(w.values, w.meta, w.scales, w.N, w.K, tv, tm)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        print(f"[transposed-graph] replay {rep}", flush=True)
        tv.zero_()
        tm.zero_()
        slim.pack_transposed(wo)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tv, ref_v) and torch.equal(tm, ref_m), f"replay {rep}"
