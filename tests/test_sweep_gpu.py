"""The LLaMA-2-7B decoder-block sweep (q/k/v/o, gate/up and down shapes at
256 and 2048 tokens, adapter rank 416, seed 0) against the fp64 oracle, in the
launch configuration the benchmark times.

At 2048 tokens the oracle checks sampled token rows (rows of Y are
independent), at least one in every 128-token block of the prefill tiles plus
the first and last.  One case takes its reference from the oracle's own pack
of W (compared byte for byte with the GPU's pack first), so the chain
pack -> linear is checked end to end without any GPU-made operand.  A ragged
shape (partial 128-token and 256-row tiles, at least 192 tiles, so no K split)
covers the unsplit prefill path on partial tiles."""
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


def _rows_every_block(M, seed, block=128, extra=8):
    """One random token row in every `block`-row block, `extra` more, the
    first and the last row."""
    rng = np.random.default_rng(seed)
    rows = [b + int(rng.integers(0, min(block, M - b))) for b in range(0, M, block)]
    rows += list(rng.choice(M, extra, replace=False)) + [0, M - 1]
    return np.unique(np.asarray(rows, dtype=np.int64))


def _check(env, case, sample, packed_by_oracle=False):
    torch, slim = env
    print(f"[sweep] {case.name} M={case.M} N={case.N} K={case.K} r={case.r} sample={sample} "
          f"oracle_pack={packed_by_oracle}", flush=True)
    inp = wl.make_inputs(case)
    (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
    if packed_by_oracle:
        ov, om, os_ = oracle.pack(inp.W)
        assert np.array_equal(v, ov) and np.array_equal(m, om), "GPU pack differs from the oracle's"
        assert np.array_equal(s.view(np.uint16), os_.view(np.uint16)), "GPU scales differ from the oracle's"
        v, m, s = ov, om, os_
    Y = slim.linear(to_dev(inp.X, torch), w, to_dev(inp.L.T, torch), to_dev(inp.R.T, torch))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    rows = _rows_every_block(case.M, case.seed + case.N + case.K) if sample else None
    ref = oracle.linear(inp.X, v, m, s, inp.L, inp.R, rows=rows)
    if rows is not None:
        Y = Y[rows]
    return assert_close_to_oracle(Y, ref, case.name)


SWEEP = [("q_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("down_proj", 4096, 11008)]


@pytest.mark.parametrize("name,N,K", SWEEP, ids=[s[0] for s in SWEEP])
def test_sweep_256_tokens(env, name, N, K):
    case = wl.Case(f"{name}@M256", M=256, N=N, K=K, r=wl.RANK)
    _check(env, case, sample=False)


@pytest.mark.parametrize("name,N,K", SWEEP, ids=[s[0] for s in SWEEP])
def test_sweep_2048_tokens_sampled(env, name, N, K):
    case = wl.Case(f"{name}@M2048", M=2048, N=N, K=K, r=wl.RANK)
    _check(env, case, sample=True)


def test_sweep_reference_from_oracle_pack(env):
    """q_proj at 256 tokens with the reference built from oracle.pack(W)."""
    case = wl.Case("q_proj@M256", M=256, N=4096, K=4096, r=wl.RANK)
    _check(env, case, sample=False, packed_by_oracle=True)


def test_prefill_unsplit_ragged_tiles(env):
    """272 tiles of 256 rows x 128 tokens (the last token and row tiles
    partial): the main kernel stores Y itself, without a K split."""
    case = wl.Case("ragged_tiles", M=2000, N=4112, K=1024, r=64, seed=77)
    _check(env, case, sample=True)
