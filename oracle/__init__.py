"""CPU oracle for the MoE verify-block path: test infrastructure only (see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (accept_histogram, accept_length, argmax_first, committed_tokens, decode_bf16,  # noqa: F401
                         decode_mxfp4, decode_tensor, expert_ffn, head_accept, head_logits, moe_block, moe_stack,
                         rms_norm, router_logits, routing_weights, sample_inverse_cdf, select_topk, silu,
                         softmax_temp, speculative_accept, topk_gap,
                         woken_experts)
from .layout import tile_bf16, tile_mxfp4, tiled_position_bf16  # noqa: F401,E402
