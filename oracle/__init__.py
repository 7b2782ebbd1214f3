"""CPU oracle of the MoE layer forward (fp64 numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU package.  Every function
cites the passage of the pages it follows; see ``moe_oracle`` for the
citation keys and the readings taken where the pages are silent.

Pins: every function here is checked against something other than itself in
``tests/test_oracle_*.py`` (closed forms, hand-derived fixtures, library
routines, brute force, invariants).  Parity unpinned: none of the pages print
activations or weights of the real model, so the numerics of the released
checkpoint itself cannot be pinned; the noaux_tc bias placement and the FP8
scale convention are readings, pinned only for self-consistency.
"""
from .moe_oracle import (E4M3_MAX, E4M3_TABLE, FP8_BLOCK, Dispatch, LayerResult, Routing,
                         Weights, block_forward, block_inputs, combine, decode_bf16,
                         decode_e4m3, dense_layer_forward, dequantize_fp8_rows,
                         dequantize_fp8_weight, dispatch, encode_bf16, encode_e4m3,
                         expert_forward, group_scores, layer_forward, layer_inputs,
                         quantize_fp8_rows, rms, rmsnorm, route, route_inputs, sigmoid,
                         selection_weights, sorted_expert_rows, swiglu_hidden, widen,
                         with_selection)

__all__ = [n for n in dir() if not n.startswith("_")]
