"""SLiM compressed linear layer on AMD Instinct MI355X (gfx950).

Y = X . deq(W_c)^T + (X . L) . R, where W_c is W quantised to symmetric int4
with fp16 scales per 128 input columns and pruned to 2:4 along the input
dimension (Compression Trinity thesis, Fig. 7.1 caption; §2.2.3).  All
computation runs in the HIP kernels of ``libslim.so``; this package only
allocates tensors with PyTorch and marshals arguments to the C ABI.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (SlimError, slim_adapter_codes_bytes, slim_adapter_scales_bytes, slim_linear,
                   slim_linear_batched, slim_linear_qa, slim_linear_qa_workspace_bytes,
                   slim_linear_workspace_bytes, slim_meta_bytes, slim_pack, slim_pack_adapter,
                   slim_pack_transposed, slim_scales_bytes, slim_transposed_meta_bytes,
                   slim_transposed_values_bytes, slim_values_bytes, slim_linear_giveups,
                   slim_set_wait_limit, slim_quantize_input, slim_linear_a8_workspace_bytes, slim_linear_a8,
                   slim_pack_hybrid, slim_linear_hybrid)

GROUP = 128

__all__ = ["SlimError", "slim_pack", "slim_linear", "slim_linear_batched",
           "slim_linear_workspace_bytes", "slim_values_bytes", "slim_meta_bytes",
           "slim_scales_bytes", "pack", "linear", "workspace", "PackedWeight",
           "slim_pack_adapter", "slim_linear_qa", "slim_linear_qa_workspace_bytes",
           "slim_adapter_codes_bytes", "slim_adapter_scales_bytes", "QuantizedAdapters",
           "pack_adapters", "workspace_qa", "linear_qa", "slim_pack_transposed",
           "slim_transposed_values_bytes", "slim_transposed_meta_bytes", "pack_transposed",
           "slim_linear_giveups", "slim_set_wait_limit", "slim_quantize_input", "slim_linear_a8_workspace_bytes",
           "slim_linear_a8", "quantize_input", "linear_a8", "slim_pack_hybrid", "slim_linear_hybrid",
           "HybridWeight", "pack_hybrid", "linear_hybrid"]

GROUP_L = 128          # quantised Lt: groups along K
GROUP_R = 32           # quantised Rt: groups along r


class PackedWeight:
    """The packed triple of one weight W [N, K] (device tensors)."""

    def __init__(self, values: torch.Tensor, meta: torch.Tensor, scales: torch.Tensor, N: int, K: int):
        self.values, self.meta, self.scales, self.N, self.K = values, meta, scales, N, K

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.values, self.meta, self.scales))


def pack(W: torch.Tensor, stream=None) -> PackedWeight:
    """Quantise, 2:4-prune and pack a float32 weight W [N, K] on the GPU."""
    if W.dtype != torch.float32:
        raise TypeError("W must be float32")
    N, K = W.shape
    dev = W.device
    # Flat buffers: the packed arrays are in 16-row blocks, group by group
    # (the layout slim.h documents), not in row order.
    values = torch.empty((N * K // 4,), dtype=torch.uint8, device=dev)
    meta = torch.empty((N * K // 8,), dtype=torch.uint8, device=dev)
    scales = torch.empty((N * K // GROUP,), dtype=torch.float16, device=dev)
    slim_pack(W, values, meta, scales, stream=stream)
    return PackedWeight(values, meta, scales, N, K)


def workspace(M: int, N: int, K: int, r: int, device="cuda", batch: int = 1) -> torch.Tensor:
    """A zero-filled workspace large enough for ``batch`` problems of this shape."""
    nbytes = slim_linear_workspace_bytes(M, N, K, r) * batch
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def linear(X: torch.Tensor, w: PackedWeight, Lt: torch.Tensor | None, Rt: torch.Tensor | None,
           ws: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X deq(W_c)^T + (X L) R with fp16 input/output.

    The adapter is given output-major: Lt = L^T [r, K], Rt = R^T [N, r]."""
    if X.dtype != torch.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    r = 0 if Lt is None else Lt.shape[0]
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=X.device)
    if ws is None:
        ws = workspace(M, w.N, K, r, device=X.device)
    slim_linear(X, w.values, w.meta, w.scales, Lt, Rt, out, ws, stream=stream)
    return out


class QuantizedAdapters:
    """int4 codes and fp16 scales of Lt = L^T [r, K] and Rt = R^T [N, r]."""

    def __init__(self, lq, ls, rq, rs, r: int, K: int, N: int):
        self.lq, self.ls, self.rq, self.rs, self.r, self.K, self.N = lq, ls, rq, rs, r, K, N

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.lq, self.ls, self.rq, self.rs))


def pack_adapters(Lt: torch.Tensor, Rt: torch.Tensor, stream=None) -> QuantizedAdapters:
    """Quantise the float32 adapter factors Lt [r, K] and Rt [N, r] on the GPU."""
    if Lt.dtype != torch.float32 or Rt.dtype != torch.float32:
        raise TypeError("Lt and Rt must be float32")
    r, K = Lt.shape
    N = Rt.shape[0]
    dev = Lt.device
    lq = torch.empty((r * K // 2,), dtype=torch.uint8, device=dev)
    ls = torch.empty((r * K // GROUP_L,), dtype=torch.float16, device=dev)
    rq = torch.empty((N * r // 2,), dtype=torch.uint8, device=dev)
    rs = torch.empty((N * r // GROUP_R,), dtype=torch.float16, device=dev)
    slim_pack_adapter(Lt, lq, ls, GROUP_L, stream=stream)
    slim_pack_adapter(Rt, rq, rs, GROUP_R, stream=stream)
    return QuantizedAdapters(lq, ls, rq, rs, r, K, N)


def workspace_qa(M: int, N: int, K: int, r: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for slim_linear_qa of this shape."""
    return torch.zeros(max(slim_linear_qa_workspace_bytes(M, N, K, r), 16), dtype=torch.uint8, device=device)


def linear_qa(X: torch.Tensor, w: PackedWeight, qa: QuantizedAdapters, ws: torch.Tensor | None = None,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X deq(W_c)^T + (X deq(L)) deq(R) with fp16 input/output."""
    if X.dtype != torch.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=X.device)
    if ws is None:
        ws = workspace_qa(M, w.N, K, qa.r, device=X.device)
    slim_linear_qa(X, w.values, w.meta, w.scales, qa.lq, qa.ls, qa.rq, qa.rs, qa.r, out, ws, stream=stream)
    return out


def pack_transposed(w: PackedWeight, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Double-pruned transpose of a packed weight (SLoPe's backward operand):
    returns (tvalues float16 [K, N/2], tmeta int16 [K, N/16]); the metadata
    half-words are uint16 bit patterns held in int16."""
    dev = w.values.device
    tvalues = torch.empty((w.K, w.N // 2), dtype=torch.float16, device=dev)
    tmeta = torch.empty((w.K, max(w.N // 16, 1)), dtype=torch.int16, device=dev)
    slim_pack_transposed(w.values, w.meta, w.scales, w.N, w.K, tvalues, tmeta, stream=stream)
    return tvalues, tmeta


def quantize_input(X: torch.Tensor, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-token int8 quantisation of fp16 X [M, K] on the GPU: (q int8 [M, K], s fp16 [M])."""
    if X.dtype != torch.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    s = torch.empty((max(M, 8),), dtype=torch.float16, device=X.device)[:M]
    slim_quantize_input(X, q, s, stream=stream)
    return q, s


def linear_a8(qx: torch.Tensor, sx: torch.Tensor, w: PackedWeight, Lt: torch.Tensor | None,
              Rt: torch.Tensor | None, ws: torch.Tensor | None = None, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Y = deq(X) deq(W_c)^T + (deq(X) L) R on an 8-bit input (qx int8 [M, K], sx fp16 [M])."""
    M, K = qx.shape
    r = 0 if Lt is None else Lt.shape[0]
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=qx.device)
    if ws is None:
        ws = torch.zeros(max(slim_linear_a8_workspace_bytes(M, w.N, K, r), 16), dtype=torch.uint8, device=qx.device)
    slim_linear_a8(qx, sx, w.values, w.meta, w.scales, Lt, Rt, out, ws, stream=stream)
    return out


class HybridWeight(PackedWeight):
    """A hybrid dense / 2:4 packed weight: the packed triple, the second pair
    of codes of dense tiles (dvalues) and the int32 tile flags [N/16, K/128]."""

    def __init__(self, values, meta, scales, dvalues, dense, N: int, K: int):
        super().__init__(values, meta, scales, N, K)
        self.dvalues, self.dense = dvalues, dense


def pack_hybrid(W: torch.Tensor, dense: torch.Tensor, stream=None) -> HybridWeight:
    """Hybrid pack of float32 W [N, K] with int32 tile flags [ceil(N/16), K/128]."""
    if W.dtype != torch.float32 or dense.dtype != torch.int32:
        raise TypeError("W must be float32 and the tile flags int32")
    N, K = W.shape
    dev = W.device
    values = torch.empty((N * K // 4,), dtype=torch.uint8, device=dev)
    meta = torch.empty((N * K // 8,), dtype=torch.uint8, device=dev)
    scales = torch.empty((N * K // GROUP,), dtype=torch.float16, device=dev)
    dvalues = torch.empty((N * K // 4,), dtype=torch.uint8, device=dev)
    dense = dense.contiguous()
    slim_pack_hybrid(W, dense, values, meta, scales, dvalues, stream=stream)
    return HybridWeight(values, meta, scales, dvalues, dense, N, K)


def linear_hybrid(X: torch.Tensor, w: HybridWeight, Lt: torch.Tensor | None, Rt: torch.Tensor | None,
                  ws: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X deq(W_h)^T + (X L) R on a hybrid dense / 2:4 weight."""
    if X.dtype != torch.float16:
        raise TypeError("X must be float16")
    M, K = X.shape
    r = 0 if Lt is None else Lt.shape[0]
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=X.device)
    if ws is None:
        ws = workspace(M, w.N, K, r, device=X.device)
    slim_linear_hybrid(X, w.values, w.meta, w.scales, w.dvalues, w.dense, Lt, Rt, out, ws, stream=stream)
    return out
