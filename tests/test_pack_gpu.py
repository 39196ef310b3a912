"""slim_pack on the GPU against the CPU oracle: bit-exact values, metadata
and scales on every workload shape and on the edge cases of the quantiser
and the 2:4 rule."""
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import sparse_int4_gemm_amd as slim
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    slim._lib.load()
    return torch, slim


def _gpu_pack(W, env):
    torch, slim = env
    w = slim.pack(to_dev(W, torch))
    torch.cuda.synchronize()
    return w.values.cpu().numpy(), w.meta.cpu().numpy(), w.scales.cpu().numpy().view(np.float16)


def _check_pack(W, env, what):
    print(f"[pack] {what} N={W.shape[0]} K={W.shape[1]}", flush=True)
    v, m, s = _gpu_pack(W, env)
    rv, rm, rs = oracle.pack(W)
    assert np.array_equal(s.view(np.uint16), rs.view(np.uint16)), f"{what}: scales differ"
    assert np.array_equal(v, rv), f"{what}: values differ"
    assert np.array_equal(m, rm), f"{what}: metadata differ"


@pytest.mark.parametrize("case", [wl.TINY, wl.QPROJ, wl.GATEUP, wl.DOWN], ids=lambda c: c.name)
def test_pack_workloads_bit_exact(env, case):
    _check_pack(wl.make_inputs(case).W, env, case.name)


def test_pack_worked_example(env, golden_dir):
    W = np.zeros((2, 128), np.float32)
    for line in open(os.path.join(golden_dir, "pack_worked_example.txt")):
        parts = line.split()
        if len(parts) == 3 and not line.startswith("#"):
            try:
                W[int(parts[0]), int(parts[1])] = np.float32(float(parts[2]))
            except ValueError:
                pass
    _check_pack(W, env, "worked example")


def test_pack_edge_cases(env):
    rng = np.random.default_rng(11)
    W = wl.random_weights(rng, 64, 1024)
    W[0] = 0.0                                         # all-zero row: s = 0, q = 0, keep (0,1)
    W[1, :128] = -0.0                                  # negative zeros
    W[2] = np.round(W[2] * 100) / 100                  # many |q| ties
    W[3, :] = np.tile([1.0, -1.0, 1.0, -1.0], 256)     # every group a 4-way tie
    W[4] *= 1e-30                                      # s16 underflows to 0
    W[5] *= 1e-4                                       # s16 subnormal in fp16
    W[6] *= 1e4                                        # large magnitudes (s16 ~ 10..)
    W[7, ::128] = 7 * 60000.0                          # s16 close to the fp16 max
    W[8, 5] = 3.5; W[8, 6] = -2.5; W[8, 7] = 2.5       # exact halves after scaling
    W[9, :] = np.float32(7.0 * (1 + 2.0 ** -11))       # scale rounds half to even
    W[10, 3::4] *= 20                                  # outliers at the last slot
    _check_pack(W, env, "edge cases")


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (7, 1152), (1, 11008), (513, 384)])
def test_pack_ragged_shapes(env, N, K):
    rng = np.random.default_rng(N * 131 + K)
    _check_pack(wl.random_weights(rng, N, K), env, f"ragged {N}x{K}")


def test_pack_deterministic(env):
    W = wl.make_inputs(wl.TINY).W
    v1, m1, s1 = _gpu_pack(W, env)
    v2, m2, s2 = _gpu_pack(W, env)
    assert np.array_equal(v1, v2) and np.array_equal(m1, m2)
