"""CPU oracle for the sparse MoE layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package. The library never does.
"""
from .moe_oracle import (  # noqa: F401
    router_logits, latent_router_logits, topk_experts, topk_gates, softmax_full, expert_capacity,
    dispatch, dispatch_remap, silu, expert_ffn, experts_forward, combine, aux_loss, moe_layer,
    lora_backward, silu_grad, gate_backward, logits_backward, experts_backward,
    router_backward, moe_layer_backward,
)
