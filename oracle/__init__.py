"""CPU oracle for the Mixtral sparse-MoE layer (float64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the library or its
binding. It shares no code with the HIP path.
"""
from .moe import (NEAR_TIE_GAP, block_forward, certify, combine, dense_masked,
                  dequantize_int8, expert_ffn, forward, gate_matrix, permute, quantize_int8,
                  renormalise, renormalised_weights_for, rms_norm, route, router_logits,
                  select_topk, silu, softmax, swiglu, tokens_output, widen)

__all__ = ["NEAR_TIE_GAP", "block_forward", "certify", "combine", "dense_masked", "dequantize_int8",
           "expert_ffn", "forward", "quantize_int8",
           "gate_matrix", "permute", "renormalise", "renormalised_weights_for", "rms_norm", "route",
           "router_logits", "select_topk", "silu", "softmax", "swiglu", "tokens_output",
           "widen"]
