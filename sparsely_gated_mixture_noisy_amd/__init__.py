"""MI355X-native forward and backward passes of the sparsely-gated noisy top-k
MoE layer.

The layer runs in libmoe.so (hand-written HIP for gfx950 behind the C ABI of
include/moe.h); this package holds the build script, the ctypes binding and
the seeded synthetic input generator.  The library is loaded on first use and
its absence is an error.
"""
from .inputs import CONFIGS, MoEConfig, make_inputs, make_upstream  # noqa: F401
from ._lib import (Backward, Forward, ForwardOut, Grads, MoEError, Workspace,  # noqa: F401
                   backward, backward_workspace_size, balance_loss, draw_noise,
                   combine, expert_ffn, forward, gate, load, pack_experts, pack_gate,
                   packed_experts_size, packed_gate_size, route, workspace, workspace_size)
