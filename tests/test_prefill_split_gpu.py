"""The K-split prefill path (128 or fewer tiles of 256 rows x 128 tokens: K
split over S workgroups per tile, fp32 partials stored tile-major, then the
T reduction and the finishing kernel) against the fp64 oracle, on every
output row, at each split count the plan chooses:

  - K = 1024, 2048, 4096, 11008 at 256 tokens (S = 2, 3, 5, 8: about six
    128-k chunks per split within the one-round cap);
  - ragged tiles: M = 100 and N = 4112 (the last token tile and row tile
    partial, lanes of tokens past M and rows past N not stored);
  - no adapter (r = 0: no T blocks, no T reduction).
"""
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


@pytest.mark.parametrize("case", [
    wl.Case("split_k1024", M=256, N=4096, K=1024, r=416, seed=41),
    wl.Case("split_k2048", M=256, N=4096, K=2048, r=416, seed=42),
    wl.Case("split_k4096", M=256, N=4096, K=4096, r=416, seed=43),
    wl.Case("split_k11008", M=256, N=1024, K=11008, r=128, seed=44),
    wl.Case("split_ragged", M=100, N=4112, K=2048, r=64, seed=45),
    wl.Case("split_r0", M=200, N=2048, K=4096, r=0, seed=46),
], ids=lambda c: c.name)
def test_prefill_split_shapes(env, case):
    torch, slim = env
    print(f"[split] {case.name} M={case.M} N={case.N} K={case.K} r={case.r}", flush=True)
    inp = wl.make_inputs(case)
    (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
    L, R = (inp.L, inp.R) if case.r > 0 else (None, None)
    Y = slim.linear(to_dev(inp.X, torch), w, None if L is None else to_dev(L.T, torch),
                    None if R is None else to_dev(R.T, torch))
    torch.cuda.synchronize()
    ref = oracle.linear(inp.X, v, m, s, L, R)
    assert_close_to_oracle(Y.cpu().numpy(), ref, case.name)
