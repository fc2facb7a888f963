"""MI355X-native forward pass of the sparsely-gated noisy top-k MoE layer.

The layer runs in libmoe.so (hand-written HIP for gfx950 behind the C ABI of
include/moe.h); this package holds the build script, the ctypes binding and
the seeded synthetic input generator.  The library is loaded on first use and
its absence is an error.
"""
from .inputs import CONFIGS, MoEConfig, make_inputs  # noqa: F401
from ._lib import (Forward, ForwardOut, MoEError, Workspace, balance_loss,  # noqa: F401
                   combine, expert_ffn, forward, gate, load, pack_experts, pack_gate,
                   packed_experts_size, packed_gate_size, route, workspace, workspace_size)
