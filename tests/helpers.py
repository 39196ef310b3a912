"""Shared helpers for the GPU parity tests (host-side marshalling only)."""
import numpy as np

REL_FRO_TOL = 2e-3      # ||Y - Y_ref||_F / ||Y_ref||_F
MAX_ABS_FRAC = 1e-2     # max|Y - Y_ref| <= MAX_ABS_FRAC * max|Y_ref|


def to_dev(a, torch):
    """Host array (any strides) -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


_ORACLE_PACKS = {}


def _oracle_pack(W):
    """oracle.pack of W, memoised by the bytes of W (tests reuse weights)."""
    import hashlib

    import oracle
    key = (W.shape, hashlib.sha1(np.ascontiguousarray(W).view(np.uint8)).hexdigest())
    if key not in _ORACLE_PACKS:
        if len(_ORACLE_PACKS) > 8:
            _ORACLE_PACKS.clear()
        _ORACLE_PACKS[key] = oracle.pack(W)
    return _ORACLE_PACKS[key]


def pack_on_gpu(W, torch, slim):
    """Pack W on the GPU, require the bytes to equal oracle.pack(W), and
    return the oracle's packed triple with a weight object holding copies of
    THOSE arrays on the device: a linear test then checks pack -> linear end
    to end, and its reference never takes a GPU-made operand."""
    w = slim.pack(to_dev(W, torch))
    torch.cuda.synchronize()
    gv, gm, gs = w.values.cpu().numpy(), w.meta.cpu().numpy(), w.scales.cpu().numpy()
    ov, om, os_ = _oracle_pack(W)
    assert np.array_equal(gv, ov), "GPU pack: values differ from the oracle's"
    assert np.array_equal(gm, om), "GPU pack: metadata differ from the oracle's"
    assert np.array_equal(gs.view(np.uint16), os_.view(np.uint16)), "GPU pack: scales differ from the oracle's"
    wo = slim.PackedWeight(to_dev(ov, torch), to_dev(om, torch), to_dev(os_.view(np.float16), torch),
                           w.N, w.K)
    return (ov, om, os_.view(np.float16)), wo


def assert_close_to_oracle(Y, Y_ref, what=""):
    Y = np.asarray(Y, dtype=np.float64)
    Y_ref = np.asarray(Y_ref, dtype=np.float64)
    assert Y.shape == Y_ref.shape, (Y.shape, Y_ref.shape)
    assert np.all(np.isfinite(Y)), f"{what}: non-finite output"
    den = np.linalg.norm(Y_ref)
    err = np.linalg.norm(Y - Y_ref)
    rel = err / den if den > 0 else err
    mx = np.max(np.abs(Y - Y_ref)) if Y.size else 0.0
    ref_mx = np.max(np.abs(Y_ref)) if Y.size else 0.0
    assert rel <= REL_FRO_TOL, f"{what}: rel Frobenius error {rel:.3e} > {REL_FRO_TOL}"
    assert mx <= MAX_ABS_FRAC * ref_mx + 1e-30, f"{what}: max|err| {mx:.3e} > {MAX_ABS_FRAC}*{ref_mx:.3e}"
    return rel, mx
