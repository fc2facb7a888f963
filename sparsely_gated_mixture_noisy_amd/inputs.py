"""Seeded synthetic inputs for the MoE layer forward.

This module holds the workload shapes and draws every tensor the layer
consumes: activations, gate tables, expert tables, the per-expert bias of the
load-skewed workload, and the standard-normal noise that noisy gating draws
(passed in as an input so that both implementations see the same draw).  It
contains none of the layer's arithmetic, and it is the only module shared by
the HIP path and the oracle.

Distributions follow the MoE lesson page ("MoE:稀疏门控混合专家"): expert FFNs
of 512 -> 1024 -> 512 (section 二), 16 groups x 256 experts for the "-h"
hierarchy (section 三), and a noise draw that is a fresh standard normal
(section 四).  Scales that the pages leave open are fixed here: activations
N(0,1), gate tables N(0, 0.02^2), expert tables N(0, 1/fan_in).

Every tensor comes from its own generator stream, seeded from (seed, tensor
name, chunk), so one tensor can be drawn without drawing the others and large
tables are drawn one expert at a time.  The values depend on the device's
generator (torch CPU and HIP generators differ); callers that compare two
implementations always hand both the very same tensors.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["MoEConfig", "CONFIGS", "make_inputs", "make_upstream", "stream_seed"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Shape and options of one MoE layer workload.

    n_groups == 0 means flat gating over n_experts; otherwise the gate picks
    k_groups of n_groups groups, then k_per_group experts inside each chosen
    group, and top_k == k_groups * k_per_group.
    """

    name: str
    tokens: int
    d_model: int
    n_experts: int
    d_hidden: int
    top_k: int
    noisy: bool = True
    ffn: str = "relu"          # "relu" or "swiglu"
    dtype: str = "bf16"        # "f32" or "bf16"
    n_groups: int = 0
    k_groups: int = 0
    k_per_group: int = 0
    bias: str = "none"         # "none" or "zipf"
    gate_std: float = 0.02
    capacity: int = 0          # rows an expert takes at most (0: no limit)

    @property
    def hierarchical(self) -> bool:
        return self.n_groups > 0

    @property
    def experts_per_group(self) -> int:
        return self.n_experts // self.n_groups if self.n_groups else self.n_experts

    @property
    def assignments(self) -> int:
        return self.tokens * self.top_k

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny fp32 check, the paper-shaped 256-expert layer,
# the 4096-expert hierarchical layer, a load-skewed 2048-expert layer and a
# Mixtral-shaped SwiGLU layer.
CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", tokens=256, d_model=64, n_experts=8, d_hidden=128,
                      top_k=2, noisy=True, dtype="f32"),
    "flat256": MoEConfig("flat256", tokens=8192, d_model=512, n_experts=256,
                         d_hidden=1024, top_k=4, noisy=True),
    "hier4096": MoEConfig("hier4096", tokens=16384, d_model=512, n_experts=4096,
                          d_hidden=1024, top_k=4, noisy=True, n_groups=16,
                          k_groups=2, k_per_group=2),
    "zipf2048": MoEConfig("zipf2048", tokens=32768, d_model=512, n_experts=2048,
                          d_hidden=1024, top_k=2, noisy=True, bias="zipf"),
    "mixtral": MoEConfig("mixtral", tokens=8192, d_model=4096, n_experts=8,
                         d_hidden=14336, top_k=2, noisy=False, ffn="swiglu"),
}

ZIPF_EXPONENT = 1.1
ZIPF_SCALE = 3.0


def stream_seed(seed: int, name: str, chunk: int = 0) -> int:
    """A 63-bit seed for the generator stream of one tensor (or one chunk)."""
    h = hashlib.sha256(f"{seed}:{name}:{chunk}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int, name: str, chunk: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, name, chunk))
    return g


def _normal(shape, std, device, seed, name, dtype, chunk=0) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed, name, chunk),
                    device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _expert_table(n, rows, cols, std, device, seed, name, dtype) -> torch.Tensor:
    """[n][rows][cols] table drawn one expert (chunk) at a time."""
    out = torch.empty((n, rows, cols), device=device, dtype=dtype)
    for e in range(n):
        out[e] = _normal((rows, cols), std, device, seed, name, dtype, chunk=e)
    return out


def zipf_bias(n_experts: int, seed: int) -> np.ndarray:
    """Per-expert logit bias for the load-skewed workload.

    z_e ~ Zipf(1.1) iid; bias_e = 3.0 * ln z_e / max_e ln z_e.  Experts with
    z_e = 1 get bias 0 and the one with the largest draw gets +3.0, which makes
    a few experts receive tens of times the mean number of tokens while many
    receive none.
    """
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, "zipf")))
    z = rng.zipf(ZIPF_EXPONENT, size=n_experts).astype(np.float64)
    lz = np.log(z)
    top = lz.max()
    if top <= 0.0:
        return np.zeros(n_experts, dtype=np.float32)
    return (ZIPF_SCALE * lz / top).astype(np.float32)


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu",
                with_experts: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Draw every input tensor of one layer call.

    Layouts (row-major):
      x          [T][d]            activations (cfg dtype)
      w_gate     [E][d]            gate table, one row per expert (the pages'
                                   d x n table stored transposed)
      w_noise    [E][d]            noise table (None when not noisy)
      bias       [E] fp32          per-expert logit bias (None unless zipf)
      eps        [T][E] fp32       noise draw (flat, noisy); for the hierarchy
                                   [T][G][E/G], read only for chosen groups
      w_gate_p   [G][d]            primary (group) gate table, hierarchy only
      w_noise_p  [G][d]            primary noise table, hierarchy only
      eps_p      [T][G] fp32       primary noise draw, hierarchy only
      w1         [E][h][d]         first expert layer (ReLU: in; SwiGLU: gate)
      w3         [E][h][d]         SwiGLU up projection (None for ReLU)
      w2         [E][d][h]         second expert layer (out / down)
    """
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    T, d, E, h = cfg.tokens, cfg.d_model, cfg.n_experts, cfg.d_hidden
    gs = cfg.gate_std
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((T, d), 1.0, device, seed, "x", dt)
    out["w_gate"] = _normal((E, d), gs, device, seed, "w_gate", dt)
    out["w_noise"] = (_normal((E, d), gs, device, seed, "w_noise", dt)
                      if cfg.noisy else None)
    if cfg.hierarchical:
        G, Eg = cfg.n_groups, cfg.experts_per_group
        out["w_gate_p"] = _normal((G, d), gs, device, seed, "w_gate_p", dt)
        out["w_noise_p"] = (_normal((G, d), gs, device, seed, "w_noise_p", dt)
                            if cfg.noisy else None)
        out["eps_p"] = (_normal((T, G), 1.0, device, seed, "eps_p", torch.float32)
                        if cfg.noisy else None)
        out["eps"] = (_normal((T, G, Eg), 1.0, device, seed, "eps", torch.float32)
                      if cfg.noisy else None)
    else:
        out["w_gate_p"] = out["w_noise_p"] = out["eps_p"] = None
        out["eps"] = (_normal((T, E), 1.0, device, seed, "eps", torch.float32)
                      if cfg.noisy else None)
    if cfg.bias == "zipf":
        out["bias"] = torch.from_numpy(zipf_bias(E, seed)).to(device)
    else:
        out["bias"] = None
    if with_experts:
        s1 = 1.0 / math.sqrt(d)
        s2 = 1.0 / math.sqrt(h)
        out["w1"] = _expert_table(E, h, d, s1, device, seed, "w1", dt)
        out["w3"] = (_expert_table(E, h, d, s1, device, seed, "w3", dt)
                     if cfg.ffn == "swiglu" else None)
        out["w2"] = _expert_table(E, d, h, s2, device, seed, "w2", dt)
    return out


def make_upstream(cfg: MoEConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    """The gradient flowing into the layer output from above, dy [T][d] ~ N(0,1)
    in the layer's dtype, for the backward pass."""
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    return _normal((cfg.tokens, cfg.d_model), 1.0, device, seed, "dy", dt)
