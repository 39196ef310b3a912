"""Shared helpers for the GPU parity tests (host-side marshalling only)."""
import numpy as np

REL_FRO_TOL = 2e-3      # ||Y - Y_ref||_F / ||Y_ref||_F
MAX_ABS_FRAC = 1e-2     # max|Y - Y_ref| <= MAX_ABS_FRAC * max|Y_ref|


def to_dev(a, torch):
    """Host array (any strides) -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def pack_on_gpu(W, torch, slim):
    w = slim.pack(to_dev(W, torch))
    torch.cuda.synchronize()
    return (w.values.cpu().numpy(), w.meta.cpu().numpy(),
            w.scales.cpu().numpy().view(np.float16)), w


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
