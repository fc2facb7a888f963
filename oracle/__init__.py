"""CPU oracle of the noisy top-k MoE layer forward (float64 numpy).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline leg may import it.  The HIP path never calls it and shares no code
with it.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (cv_squared, combine, dense_forward, dense_gates,  # noqa: F401
                         expert_relu, expert_swiglu, flat_gate, forward, gate,
                         hier_gate, importance, keep_top_k, kept_softmax,
                         load_estimate, noisy_logits, normal_cdf, route,
                         run_experts, silu, softplus,
                         balance_stats, backward, cv_squared_grad, rank_experts,
                         expert_relu_backward, expert_swiglu_backward, normal_pdf,
                         sigmoid, philox4x32_10, uniform23, philox_normals, draw_noise,
                         batch_mask, threshold_mask, masked_gates, masked_route,
                         masked_forward)
