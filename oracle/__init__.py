"""Float64 CPU oracle for the MXFP4 grouped-expert MoE layer (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use it.
"""
from .moe_oracle import (E2M1_VALUES, bf16_to_f64, decode_e2m1, decode_e8m0,
                         unpack_codes, dequant_mxfp4, blocked_from_canonical,
                         canonical_from_blocked, router_logits, top_k,
                         softmax_selected, sigmoid_selected, GATINGS, route,
                         build_tiles, silu, expert_ffn, combine, moe_layer,
                         GPTOSS_ALPHA, GPTOSS_LIMIT, concatenated_from_interleaved,
                         swiglu_clamped, expert_ffn_gptoss)

__all__ = ["E2M1_VALUES", "bf16_to_f64", "decode_e2m1", "decode_e8m0", "unpack_codes",
           "dequant_mxfp4", "blocked_from_canonical", "canonical_from_blocked",
           "router_logits", "top_k", "softmax_selected", "sigmoid_selected", "GATINGS", "route",
           "build_tiles", "silu", "expert_ffn", "combine", "moe_layer", "GPTOSS_ALPHA",
           "GPTOSS_LIMIT", "concatenated_from_interleaved", "swiglu_clamped",
           "expert_ffn_gptoss"]
