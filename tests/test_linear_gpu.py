"""slim_linear / slim_linear_batched on the GPU against the fp64 CPU oracle.

Bar: relative Frobenius error <= 2e-3 and max|err| <= 1e-2 * max|y_ref|
(fp16 input/output, fp32 accumulation).  Full-size configurations are run
in the same launch configuration as the benchmark; the oracle then checks a
sample of output rows (rows of Y are independent)."""
import dataclasses

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


def _run_case(env, X, W, L, R, what, sample_rows=None):
    torch, slim = env
    print(f"[linear] {what} M={X.shape[0]} N={W.shape[0]} K={W.shape[1]} r={0 if L is None else L.shape[1]}",
          flush=True)
    (v, m, s), w = pack_on_gpu(W, torch, slim)
    dX = to_dev(X, torch)
    dL = None if L is None else to_dev(L.T, torch)      # Lt = L^T [r, K]
    dR = None if R is None else to_dev(R.T, torch)      # Rt = R^T [N, r]
    Y = slim.linear(dX, w, dL, dR)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    rows = sample_rows
    Y_ref = oracle.linear(X, v, m, s, L, R, rows=rows)
    if rows is not None:
        Y = Y[rows]
    return assert_close_to_oracle(Y, Y_ref, what)


@pytest.mark.parametrize("case", [wl.TINY, wl.QPROJ, wl.QPROJ.with_M(16), wl.GATEUP, wl.DOWN.with_M(1), wl.DOWN.with_M(2)],
                         ids=lambda c: f"{c.name}@M{c.M}")
def test_linear_workloads(env, case):
    inp = wl.make_inputs(case)
    _run_case(env, inp.X, inp.W, inp.L, inp.R, case.name)


def test_linear_down_prefill_sampled(env):
    inp = wl.make_inputs(wl.DOWN)
    rows = np.random.default_rng(0).choice(wl.DOWN.M, 48, replace=False)
    rows = np.sort(np.concatenate([rows, [0, wl.DOWN.M - 1]]))
    _run_case(env, inp.X, inp.W, inp.L, inp.R, "down@M2048 (sampled rows)", sample_rows=rows)


@pytest.mark.parametrize("M", [1, 2, 3, 15, 17, 33, 100, 255, 257, 1000])
def test_linear_ragged_M(env, M):
    case = wl.Case("ragged", M=M, N=1024, K=1024, r=64, seed=M)
    inp = wl.make_inputs(case)
    _run_case(env, inp.X, inp.W, inp.L, inp.R, f"ragged M={M}")


@pytest.mark.parametrize("N,K,r", [(16, 128, 32), (48, 384, 0), (1040, 1152, 96), (11008, 128, 32),
                                   (272, 11008, 416), (11200, 1024, 256), (8192, 2048, 192)])
def test_linear_shapes(env, N, K, r):
    for M in (1, 16, 300):
        case = wl.Case("shape", M=M, N=N, K=K, r=r, seed=N + K + r + M)
        inp = wl.make_inputs(case)
        L, R = (inp.L, inp.R) if r > 0 else (None, None)
        _run_case(env, inp.X, inp.W, L, R, f"N={N} K={K} r={r} M={M}")


def test_linear_no_adapter_and_zero_weight(env):
    case = wl.Case("z", M=16, N=256, K=512, r=32, seed=5)
    inp = wl.make_inputs(case)
    _run_case(env, inp.X, inp.W, None, None, "r=0")
    _run_case(env, inp.X, np.zeros_like(inp.W), inp.L, inp.R, "W=0 (adapter only)")


def test_linear_outliers_and_large_values(env):
    case = wl.Case("o", M=16, N=512, K=1024, r=64, seed=9, outlier_frac=0.05)
    inp = wl.make_inputs(case)
    _run_case(env, inp.X * np.float16(4), inp.W * np.float32(10), inp.L, inp.R, "outliers x10")


def test_linear_empty_M(env):
    torch, slim = env
    inp = wl.make_inputs(wl.TINY)
    _, w = pack_on_gpu(inp.W, torch, slim)
    X = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    Y = slim.linear(X, w, to_dev(inp.L.T, torch), to_dev(inp.R.T, torch))
    torch.cuda.synchronize()
    assert Y.shape == (0, 512)


def test_linear_repeatable_and_workspace_reuse(env):
    torch, slim = env
    inp = wl.make_inputs(wl.QPROJ.with_M(16))
    _, w = pack_on_gpu(inp.W, torch, slim)
    dX, dL, dR = to_dev(inp.X, torch), to_dev(inp.L.T, torch), to_dev(inp.R.T, torch)
    ws = slim.workspace(16, 4096, 4096, 416)
    Y1 = slim.linear(dX, w, dL, dR, ws=ws).cpu().numpy()
    for _ in range(3):
        Y2 = slim.linear(dX, w, dL, dR, ws=ws).cpu().numpy()
        assert np.array_equal(Y1, Y2)


@pytest.mark.parametrize("M", [16, 200])
def test_linear_batched(env, M):
    torch, slim = env
    B, N, K, r = 3, 1024, 2048, 64
    cases = [wl.Case("b", M=M, N=N, K=K, r=r, seed=100 + b) for b in range(B)]
    inps = [wl.make_inputs(c) for c in cases]
    packs = [pack_on_gpu(i.W, torch, slim) for i in inps]
    for shared_x in (False, True):
        print(f"[batched] shared_x={shared_x}", flush=True)
        X = np.stack([inps[0].X if shared_x else i.X for i in inps])
        dX = to_dev(X[:1] if shared_x else X, torch)
        dV = torch.stack([p[1].values for p in packs]).contiguous()
        dM = torch.stack([p[1].meta for p in packs]).contiguous()
        dS = torch.stack([p[1].scales for p in packs]).contiguous()
        dL = to_dev(np.stack([i.L.T for i in inps]), torch)
        dR = to_dev(np.stack([i.R.T for i in inps]), torch)
        dY = torch.empty((B, M, N), dtype=torch.float16, device="cuda")
        ws = slim.workspace(M, N, K, r, batch=B)
        slim.slim_linear_batched(B, M, N, K, r, dX, 0 if shared_x else M * K, dV, N * K // 4,
                                 dM, N * K // 8, dS, N * K // 128, dL, K * r, dR, r * N, dY, M * N, ws)
        torch.cuda.synchronize()
        Y = dY.cpu().numpy()
        for b in range(B):
            v, m, s = packs[b][0]
            ref = oracle.linear(X[b], v, m, s, inps[b].L, inps[b].R)
            assert_close_to_oracle(Y[b], ref, f"batched[{b}] shared_x={shared_x}")


def test_linear_in_captured_graph_replays(env):
    """slim_linear captured in a HIP graph: every replay (with eager work and
    synchronisations in between) equals the eager result bit for bit."""
    torch, slim = env
    for case in (wl.QPROJ, wl.QPROJ.with_M(16), wl.TINY, wl.GATEUP.with_M(1), wl.GATEUP, wl.DOWN.with_M(16)):
        print(f"[graph] {case.name}", flush=True)
        inp = wl.make_inputs(case)
        _, w = pack_on_gpu(inp.W, torch, slim)
        dX, dL, dR = to_dev(inp.X, torch), to_dev(inp.L.T, torch), to_dev(inp.R.T, torch)
        ws = slim.workspace(case.M, case.N, case.K, case.r)
        Y_eager = slim.linear(dX, w, dL, dR, ws=ws).clone()
        Y = torch.zeros_like(Y_eager)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                slim.linear(dX, w, dL, dR, ws=ws, out=Y)
        torch.cuda.current_stream().wait_stream(cap)
        for rep in range(3):
            Y.zero_()
            slim.linear(dX, w, dL, dR, ws=ws)          # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Y_eager), f"{case.name}: replay {rep} differs from eager"


def test_linear_decode_handoff_state_across_calls(env):
    """One workspace through a mixed sequence of calls: one-launch decode calls
    (one or two tokens; their workgroups exchange the rows of T through tagged
    entries and an epoch word in the reserved workspace bytes) between calls
    of other shapes and paths, each with fresh inputs.  Every result matches
    the oracle, and each one-launch call advances the epoch word by one."""
    torch, slim = env
    seq = [wl.Case("h0", M=1, N=4096, K=4096, r=416, seed=21),
           wl.Case("h1", M=2, N=1024, K=1024, r=64, seed=22),
           wl.Case("h2", M=16, N=1024, K=1024, r=64, seed=23),     # two-launch decode path
           wl.Case("h3", M=1, N=1040, K=1152, r=96, seed=24),
           wl.Case("h4", M=300, N=1024, K=1024, r=64, seed=25),    # prefill path
           wl.Case("h5", M=1, N=4096, K=4096, r=416, seed=26),
           wl.Case("h6", M=2, N=4096, K=11008, r=416, seed=27),
           wl.Case("h7", M=1, N=11008, K=4096, r=416, seed=28),   # one launch, three blocks per workgroup
           wl.Case("h8", M=16, N=11008, K=4096, r=416, seed=29),  # K split, six-block row groups
           wl.Case("h9", M=2, N=11008, K=4096, r=416, seed=30)]
    nbytes = max(slim.slim_linear_workspace_bytes(c.M, c.N, c.K, c.r) for c in seq)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    epoch = 0
    for c in seq:
        print(f"[handoff] {c.name} M={c.M} N={c.N} K={c.K} r={c.r}", flush=True)
        inp = wl.make_inputs(c)
        (v, m, s), w = pack_on_gpu(inp.W, torch, slim)
        Y = slim.linear(to_dev(inp.X, torch), w, to_dev(inp.L.T, torch), to_dev(inp.R.T, torch), ws=ws)
        torch.cuda.synchronize()
        ref = oracle.linear(inp.X, v, m, s, inp.L, inp.R)
        assert_close_to_oracle(Y.cpu().numpy(), ref, c.name)
        word = int(ws[:8].cpu().view(torch.int64).item())
        if c.M <= 2:
            epoch += 1
        assert word == epoch, f"{c.name}: epoch word {word}, expected {epoch}"
    assert slim.slim_linear_giveups(ws) == 0


# One-launch forms: T wave with one and with three row blocks per workgroup,
# the 1024-thread T wave (long K), and decode_kernel's fused form (K too long
# for the T wave's LDS layout at two tokens).
GIVEUP_CASES = [wl.QPROJ, wl.GATEUP.with_M(1), wl.DOWN.with_M(2),
                wl.Case("fused16w", M=2, N=4096, K=13312, r=416, seed=31)]


@pytest.mark.parametrize("case", GIVEUP_CASES, ids=lambda c: f"{c.name}@M{c.M}")
def test_linear_decode_giveup_is_reported_and_harmless(env, case):
    """With the wait limit at 0 every workgroup of a one-launch decode call
    gives up at once (forced from the host; every kernel exits normally): its
    rows of Y read NaN, the workspace's give-up count reports it, and the next
    call on the same workspace, with other inputs and the default limit,
    matches the oracle (no entry of the failed call is taken for its own)."""
    torch, slim = env
    print(f"[giveup] {case.name} M={case.M} N={case.N} K={case.K} r={case.r}", flush=True)
    ws = slim.workspace(case.M, case.N, case.K, case.r)
    inp = wl.make_inputs(case)
    _, w = pack_on_gpu(inp.W, torch, slim)
    prev = slim.slim_set_wait_limit(0)
    try:
        Y = slim.linear(to_dev(inp.X, torch), w, to_dev(inp.L.T, torch), to_dev(inp.R.T, torch), ws=ws)
        torch.cuda.synchronize()
    finally:
        slim.slim_set_wait_limit(prev)
    assert np.isnan(Y.float().cpu().numpy()).all(), "a workgroup that gave up must write NaN"
    n = slim.slim_linear_giveups(ws)
    assert n >= 1
    # Workgroups that give up raise the epoch to their tags; one that starts
    # after such a raise reads the raised epoch, so it may end above 1.
    e1 = int(ws[:8].cpu().view(torch.int64).item())
    assert e1 >= 1, "the give-up raises the epoch to its tag"
    # Next call: new inputs (a stale T would now give a wrong, finite Y).
    inp2 = wl.make_inputs(dataclasses.replace(case, seed=case.seed + 1000))
    (v2, m2, s2), w2 = pack_on_gpu(inp2.W, torch, slim)
    Y2 = slim.linear(to_dev(inp2.X, torch), w2, to_dev(inp2.L.T, torch), to_dev(inp2.R.T, torch), ws=ws)
    torch.cuda.synchronize()
    assert_close_to_oracle(Y2.cpu().numpy(), oracle.linear(inp2.X, v2, m2, s2, inp2.L, inp2.R), "after a give-up")
    assert int(ws[:8].cpu().view(torch.int64).item()) == e1 + 1
    assert slim.slim_linear_giveups(ws, reset=True) == n, "a completed call adds no give-up"
    assert slim.slim_linear_giveups(ws) == 0


@pytest.mark.parametrize("M", [7, 16])
def test_linear_split_eight_block_groups(env, M):
    """Row groups of eight 16-row blocks at a K split of 8 (down_proj-like
    K = 11008; 250 blocks: the last group holds two)."""
    case = wl.Case("eight", M=M, N=4000, K=11008, r=416, seed=800 + M)
    inp = wl.make_inputs(case)
    _run_case(env, inp.X, inp.W, inp.L, inp.R, f"eight-block groups M={M}")


def test_linear_down_decode_16_tokens(env):
    inp = wl.make_inputs(wl.DOWN.with_M(16))
    _run_case(env, inp.X, inp.W, inp.L, inp.R, "down@M16")


@pytest.mark.parametrize("M", [3, 9, 16])
def test_linear_split_six_block_groups(env, M):
    """3 to 16 tokens where row groups of six 16-row blocks bring the K-split
    items into one round (700 blocks: the last group holds four)."""
    case = wl.Case("six", M=M, N=11200, K=1024, r=256, seed=600 + M)
    inp = wl.make_inputs(case)
    _run_case(env, inp.X, inp.W, inp.L, inp.R, f"six-block groups M={M}")


@pytest.mark.parametrize("M", [1, 16, 300])
def test_linear_large_rank(env, M):
    """r = 640: beyond the one-launch decode (two launches at one token), the
    K-split decode's larger row groups, and the LDS-staged prefill finish
    (the finish that reads its operands from global memory runs)."""
    case = wl.Case("rank640", M=M, N=5120, K=1024, r=640, seed=640 + M)
    inp = wl.make_inputs(case)
    _run_case(env, inp.X, inp.W, inp.L, inp.R, f"r=640 M={M}")
