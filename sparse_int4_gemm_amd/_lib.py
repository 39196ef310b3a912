"""ctypes binding of libslim.so (include/slim.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI; all computation runs in the library's
HIP kernels.  PyTorch supplies device memory and streams.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SLIM_LIB", os.path.join(_HERE, "libslim.so"))

SLIM_OK = 0
SLIM_EINVAL = 1
SLIM_EUNSUPPORTED = 2
SLIM_EHIP = 3

EXPORTED = (
    "slim_status_string", "slim_last_error", "slim_version",
    "slim_values_bytes", "slim_meta_bytes", "slim_scales_bytes",
    "slim_pack", "slim_linear_workspace_bytes", "slim_linear", "slim_linear_batched",
    "slim_adapter_codes_bytes", "slim_adapter_scales_bytes", "slim_pack_adapter",
    "slim_linear_qa_workspace_bytes", "slim_linear_qa",
    "slim_transposed_values_bytes", "slim_transposed_meta_bytes", "slim_pack_transposed",
    "slim_linear_giveups", "slim_set_wait_limit", "slim_linear_noalloc",
    "slim_quantize_input", "slim_linear_a8_workspace_bytes", "slim_linear_a8",
    "slim_pack_hybrid", "slim_linear_hybrid",
)

_lib = None


class SlimError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libslim.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_int4_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, sz, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.slim_status_string.restype = ctypes.c_char_p
    lib.slim_status_string.argtypes = [ctypes.c_int]
    lib.slim_last_error.restype = ctypes.c_char_p
    lib.slim_last_error.argtypes = []
    lib.slim_version.restype = ctypes.c_int
    for f in ("slim_values_bytes", "slim_meta_bytes"):
        getattr(lib, f).restype = sz
        getattr(lib, f).argtypes = [i64, i64]
    lib.slim_scales_bytes.restype = sz
    lib.slim_scales_bytes.argtypes = [i64, i64, i64]
    lib.slim_pack.restype = ctypes.c_int
    lib.slim_pack.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    lib.slim_linear_workspace_bytes.restype = sz
    lib.slim_linear_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.slim_linear.restype = ctypes.c_int
    lib.slim_linear.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp, sz, vp]
    lib.slim_linear_batched.restype = ctypes.c_int
    lib.slim_linear_batched.argtypes = [i64, i64, i64, i64, i64, i64,
                                        vp, i64, vp, i64, vp, i64, vp, i64,
                                        vp, i64, vp, i64, vp, i64, vp, sz, vp]
    lib.slim_adapter_codes_bytes.restype = sz
    lib.slim_adapter_codes_bytes.argtypes = [i64, i64]
    lib.slim_adapter_scales_bytes.restype = sz
    lib.slim_adapter_scales_bytes.argtypes = [i64, i64, i64]
    lib.slim_pack_adapter.restype = ctypes.c_int
    lib.slim_pack_adapter.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.slim_linear_qa_workspace_bytes.restype = sz
    lib.slim_linear_qa_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.slim_linear_qa.restype = ctypes.c_int
    lib.slim_linear_qa.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, vp, vp, vp, vp, i64, vp, vp, sz, vp]
    lib.slim_transposed_values_bytes.restype = sz
    lib.slim_transposed_values_bytes.argtypes = [i64, i64]
    lib.slim_transposed_meta_bytes.restype = sz
    lib.slim_transposed_meta_bytes.argtypes = [i64, i64]
    lib.slim_pack_transposed.restype = ctypes.c_int
    lib.slim_pack_transposed.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.slim_linear_giveups.restype = ctypes.c_int
    lib.slim_linear_giveups.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64), vp]
    lib.slim_set_wait_limit.restype = i64
    lib.slim_set_wait_limit.argtypes = [i64]
    lib.slim_quantize_input.restype = ctypes.c_int
    lib.slim_quantize_input.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.slim_linear_a8_workspace_bytes.restype = sz
    lib.slim_linear_a8_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.slim_linear_a8.restype = ctypes.c_int
    lib.slim_linear_a8.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp, sz, vp]
    lib.slim_pack_hybrid.restype = ctypes.c_int
    lib.slim_pack_hybrid.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.slim_linear_hybrid.restype = ctypes.c_int
    lib.slim_linear_hybrid.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp, vp, i64, vp, vp, sz, vp]
    lib.slim_linear_noalloc.restype = ctypes.c_int
    lib.slim_linear_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != SLIM_OK:
        lib = load()
        raise SlimError(status, f"{lib.slim_status_string(status).decode()} — {lib.slim_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU (a ROCm 'cuda' device)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------- raw ABI calls
def slim_values_bytes(N: int, K: int) -> int:
    return load().slim_values_bytes(N, K)


def slim_meta_bytes(N: int, K: int) -> int:
    return load().slim_meta_bytes(N, K)


def slim_scales_bytes(N: int, K: int, group: int = 128) -> int:
    return load().slim_scales_bytes(N, K, group)


def slim_linear_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return load().slim_linear_workspace_bytes(M, N, K, r)


def slim_pack(W, values, meta, scales, group: int = 128, stream=None) -> None:
    N, K = W.shape
    _check(load().slim_pack(_ptr(W), N, K, group, _ptr(values), _ptr(meta), _ptr(scales), _stream(stream)))


def slim_linear(X, values, meta, scales, Lt, Rt, Y, workspace, group: int = 128, stream=None) -> None:
    """Lt = L^T [r, K] and Rt = R^T [N, r] (fp16); None for no adapter."""
    M, K = X.shape
    N = Y.shape[1]
    r = 0 if Lt is None else Lt.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().slim_linear(_ptr(X), M, N, K, _ptr(values), _ptr(meta), _ptr(scales), group,
                              _ptr(Lt), _ptr(Rt), r, _ptr(Y), _ptr(workspace), ws_bytes, _stream(stream)))


def slim_linear_batched(batch, M, N, K, r, X, stride_X, values, stride_values, meta, stride_meta,
                        scales, stride_scales, Lt, stride_Lt, Rt, stride_Rt, Y, stride_Y, workspace,
                        group: int = 128, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().slim_linear_batched(batch, M, N, K, r, group,
                                      _ptr(X), stride_X, _ptr(values), stride_values,
                                      _ptr(meta), stride_meta, _ptr(scales), stride_scales,
                                      _ptr(Lt), stride_Lt, _ptr(Rt), stride_Rt, _ptr(Y), stride_Y,
                                      _ptr(workspace), ws_bytes, _stream(stream)))


def slim_adapter_codes_bytes(rows: int, cols: int) -> int:
    return load().slim_adapter_codes_bytes(rows, cols)


def slim_adapter_scales_bytes(rows: int, cols: int, group: int) -> int:
    return load().slim_adapter_scales_bytes(rows, cols, group)


def slim_linear_qa_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return load().slim_linear_qa_workspace_bytes(M, N, K, r)


def slim_pack_adapter(A, codes, scales, group: int, stream=None) -> None:
    """A: fp32 factor [rows, cols] stored output-major (Lt or Rt)."""
    rows, cols = A.shape
    _check(load().slim_pack_adapter(_ptr(A), rows, cols, group, _ptr(codes), _ptr(scales), _stream(stream)))


def slim_linear_qa(X, values, meta, scales, Lq, Ls, Rq, Rs, r, Y, workspace, group: int = 128, stream=None) -> None:
    M, K = X.shape
    N = Y.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().slim_linear_qa(_ptr(X), M, N, K, _ptr(values), _ptr(meta), _ptr(scales), group,
                                 _ptr(Lq), _ptr(Ls), _ptr(Rq), _ptr(Rs), r, _ptr(Y), _ptr(workspace), ws_bytes,
                                 _stream(stream)))


def slim_transposed_values_bytes(N: int, K: int) -> int:
    return load().slim_transposed_values_bytes(N, K)


def slim_transposed_meta_bytes(N: int, K: int) -> int:
    return load().slim_transposed_meta_bytes(N, K)


def slim_pack_transposed(values, meta, scales, N: int, K: int, tvalues, tmeta, group: int = 128,
                         stream=None) -> None:
    """Double-pruned transpose of a packed W [N, K]: tvalues fp16 [K, N/2],
    tmeta uint16 [K, N/16] (int16 tensors hold the bit patterns)."""
    _check(load().slim_pack_transposed(_ptr(values), _ptr(meta), _ptr(scales), N, K, group, _ptr(tvalues),
                                       _ptr(tmeta), _stream(stream)))


def slim_linear_giveups(workspace, reset: bool = False, stream=None) -> int:
    """Workgroups of the one-launch decode path that gave up their bounded
    wait on this workspace (synchronises the stream)."""
    n = ctypes.c_uint64(0)
    _check(load().slim_linear_giveups(_ptr(workspace), 1 if reset else 0, ctypes.byref(n), _stream(stream)))
    return int(n.value)


def slim_set_wait_limit(limit: int) -> int:
    """Poll passes before a one-launch decode workgroup gives up (0: at once,
    negative: the default).  Returns the previous limit."""
    return int(load().slim_set_wait_limit(limit))


def slim_linear_noalloc(X, values, meta, scales, Lt, Rt, Y, group: int = 128, stream=None) -> None:
    """slim_linear with the library's own per-GPU scratch (no workspace)."""
    M, K = X.shape
    N = Y.shape[1]
    r = 0 if Lt is None else Lt.shape[0]
    _check(load().slim_linear_noalloc(_ptr(X), M, N, K, _ptr(values), _ptr(meta), _ptr(scales), group,
                                      _ptr(Lt), _ptr(Rt), r, _ptr(Y), _stream(stream)))


def slim_quantize_input(X, q, s, stream=None) -> None:
    """Per-token int8 quantisation of fp16 X [M, K] into q (int8 [M, K]) and s (fp16 [M])."""
    M, K = X.shape
    _check(load().slim_quantize_input(_ptr(X), M, K, _ptr(q), _ptr(s), _stream(stream)))


def slim_linear_a8_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return load().slim_linear_a8_workspace_bytes(M, N, K, r)


def slim_linear_a8(qx, sx, values, meta, scales, Lt, Rt, Y, workspace, group: int = 128, stream=None) -> None:
    """The layer on an 8-bit input: qx int8 [M, K], sx fp16 [M]."""
    M, K = qx.shape
    N = Y.shape[1]
    r = 0 if Lt is None else Lt.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().slim_linear_a8(_ptr(qx), _ptr(sx), M, N, K, _ptr(values), _ptr(meta), _ptr(scales), group,
                                 _ptr(Lt), _ptr(Rt), r, _ptr(Y), _ptr(workspace), ws_bytes, _stream(stream)))


def slim_pack_hybrid(W, dense, values, meta, scales, dvalues, group: int = 128, stream=None) -> None:
    """Hybrid dense / 2:4 pack; dense: int32 [ceil(N/16), K/128] tile flags."""
    N, K = W.shape
    _check(load().slim_pack_hybrid(_ptr(W), N, K, group, _ptr(dense), _ptr(values), _ptr(meta), _ptr(scales),
                                   _ptr(dvalues), _stream(stream)))


def slim_linear_hybrid(X, values, meta, scales, dvalues, dense, Lt, Rt, Y, workspace, group: int = 128,
                       stream=None) -> None:
    M, K = X.shape
    N = Y.shape[1]
    r = 0 if Lt is None else Lt.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().slim_linear_hybrid(_ptr(X), M, N, K, _ptr(values), _ptr(meta), _ptr(scales), _ptr(dvalues),
                                     _ptr(dense), group, _ptr(Lt), _ptr(Rt), r, _ptr(Y), _ptr(workspace), ws_bytes,
                                     _stream(stream)))
