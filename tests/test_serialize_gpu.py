"""The packed triple (values, meta, scales) with Lt and Rt is the serialized
compressed layer: saved with torch.save or as raw bytes and loaded back, it
must give a bit-identical Y.  Every path is also deterministic: the same call
twice gives the same bits (the reductions are two-stage, never fp32 atomics).
Shapes: one token (one-launch decode), 16 tokens (K-split decode), 256 tokens
(K-split prefill) and 2048 tokens (one-pass prefill)."""
import numpy as np
import pytest

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


@pytest.mark.parametrize("M", [1, 16, 256, 2048])
def test_save_load_gives_identical_output(env, tmp_path, M):
    torch, slim = env
    case = wl.Case("ser", M=M, N=4096, K=1024, r=64, seed=70 + M)
    print(f"[serialize] M={M} N={case.N} K={case.K} r={case.r}", flush=True)
    inp = wl.make_inputs(case)
    w = slim.pack(to_dev(inp.W, torch))
    X = to_dev(inp.X, torch)
    Lt, Rt = to_dev(inp.L.T, torch), to_dev(inp.R.T, torch)
    Y0 = slim.linear(X, w, Lt, Rt).cpu().numpy()
    Y1 = slim.linear(X, w, Lt, Rt).cpu().numpy()
    assert np.array_equal(Y0.view(np.uint16), Y1.view(np.uint16)), "two identical calls differ"

    # torch.save / torch.load (tensor data only)
    path = tmp_path / "layer.pt"
    torch.save({"values": w.values.cpu(), "meta": w.meta.cpu(), "scales": w.scales.cpu(),
                "Lt": Lt.cpu(), "Rt": Rt.cpu(), "N": w.N, "K": w.K}, path)
    d = torch.load(path, weights_only=True)
    w2 = slim.PackedWeight(d["values"].cuda(), d["meta"].cuda(), d["scales"].cuda(), d["N"], d["K"])
    Y2 = slim.linear(X, w2, d["Lt"].cuda(), d["Rt"].cuda()).cpu().numpy()
    assert np.array_equal(Y0.view(np.uint16), Y2.view(np.uint16)), "reloaded layer (torch.save) differs"

    # raw bytes
    arrays = {"values": w.values, "meta": w.meta, "scales": w.scales, "Lt": Lt, "Rt": Rt}
    loaded = {}
    for name, t in arrays.items():
        host = t.cpu().numpy()
        f = tmp_path / f"{name}.bin"
        host.tofile(f)
        back = np.fromfile(f, dtype=host.dtype).reshape(host.shape)
        assert np.array_equal(back.view(np.uint8), host.view(np.uint8))
        loaded[name] = to_dev(back, torch)
    w3 = slim.PackedWeight(loaded["values"], loaded["meta"], loaded["scales"], w.N, w.K)
    Y3 = slim.linear(X, w3, loaded["Lt"], loaded["Rt"]).cpu().numpy()
    assert np.array_equal(Y0.view(np.uint16), Y3.view(np.uint16)), "reloaded layer (raw bytes) differs"
