"""CPU oracle for the SLiM compressed linear layer.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The GPU library does not use
it, and it shares no code with the GPU path.

Pins: every function here is checked against facts that the method's pages and
plain mathematics fix (see tests/test_oracle.py); no function is
"parity unpinned".
"""
from .slim_ref import (ADAPTER_GROUP_L, ADAPTER_GROUP_R, GROUP, NIB_POS, QMAX, arrange, dequantize,
                       dequantized_adapters, encode, group_scales, linear, linear_batched, linear_qa, pack,
                       pack_adapter, pack_adapters, pack_rows, pack_transposed, prune_2of4, quantize,
                       quantize_adapter, rows_of, unpack, unpack_adapter, unpack_transposed,
                       QMAX_INPUT, dequantize_input, linear_a8, quantize_input,
                       TILE_ROWS, expand_tile_flags, linear_hybrid, pack_hybrid, unpack_hybrid)

__all__ = ["GROUP", "QMAX", "group_scales", "quantize", "prune_2of4", "encode",
           "arrange", "rows_of", "pack_rows", "pack", "unpack", "dequantize", "linear",
           "linear_batched", "ADAPTER_GROUP_L", "ADAPTER_GROUP_R", "NIB_POS", "quantize_adapter",
           "pack_adapter", "unpack_adapter", "pack_adapters", "dequantized_adapters", "linear_qa",
           "pack_transposed", "unpack_transposed", "QMAX_INPUT", "quantize_input", "dequantize_input",
           "linear_a8", "TILE_ROWS", "expand_tile_flags", "pack_hybrid", "unpack_hybrid", "linear_hybrid"]
