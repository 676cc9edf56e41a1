"""The five workload shapes of the fused MoE layer, plus a helper for small
variants used by tests.

Shapes and distributions:
  tiny_fp32            T=64,    H=128,  I=256,  E=8,   K=2, renormalised, f32
  qwen2_moe_bf16       T=4096,  H=2048, I=1408, E=60,  K=4, not renormalised
  deepseek_v2_bf16     T=8192,  H=5120, I=1536, E=160, K=6, per-expert logit
                       bias ~ N(0, 0.5) for moderately skewed load
  ep_share_256_bf16    T=8192,  H=2048, I=512,  E=256, K=8, 4 EP ranks of 64
                       experts each (one rank's share per call)
  redundant_slots_zipf T=16384, H=4096, I=1024, E=64 in S=80 slots, K=8; the
                       16 most popular experts get a second slot; expert
                       popularity follows Zipf(s=1.2)

Readings: the second parameter of N(mu, sigma) is a standard deviation; where
the renormalisation flag is not stated the module default (renormalise) is
taken, following the FusedMoE constructor's renormalize=True default in vLLM
ep_fused_moe_patch.py.
"""
from __future__ import annotations

import dataclasses
from typing import Optional


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    T: int
    H: int
    I: int
    E: int          # global routed experts
    K: int
    renormalize: bool
    dtype: str      # "f32", "bf16" or "fp8" (bf16 input, E4M3 expert weights)
    router: str     # "gauss", "gauss_bias", "zipf"
    ep_size: int = 1
    n_replicated: int = 0     # experts given a second slot (zipf workload)
    bias_std: float = 0.0     # per-expert logit bias std (gauss_bias)
    zipf_s: float = 1.2
    seed: int = 0
    num_expert_group: int = 0  # group-limited routing: groups (0 = plain top-K)
    topk_group: int = 0        # groups kept
    shared_expert: bool = False     # a shared-expert output [T, H] is added in the combine
    routing_on_input: bool = False  # routing weights applied to the expert input
    a1_scale: float = 1.0 / 56.0    # fp8: scale of the quantized expert input (x ~ N(0,1))
    a2_scale: float = 1.0 / 14.0    # fp8: scale of the quantized SwiGLU output

    @property
    def E_local(self) -> int:
        return self.E // self.ep_size

    @property
    def S(self) -> int:
        """Slots held by one share."""
        return self.E_local + self.n_replicated

    @property
    def pairs(self) -> int:
        return self.T * self.K

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    c.name: c
    for c in [
        WorkloadConfig("tiny_fp32", T=64, H=128, I=256, E=8, K=2, renormalize=True,
                       dtype="f32", router="gauss"),
        WorkloadConfig("qwen2_moe_bf16", T=4096, H=2048, I=1408, E=60, K=4,
                       renormalize=False, dtype="bf16", router="gauss"),
        WorkloadConfig("deepseek_v2_bf16", T=8192, H=5120, I=1536, E=160, K=6,
                       renormalize=True, dtype="bf16", router="gauss_bias", bias_std=0.5),
        WorkloadConfig("ep_share_256_bf16", T=8192, H=2048, I=512, E=256, K=8,
                       renormalize=True, dtype="bf16", router="gauss", ep_size=4),
        WorkloadConfig("redundant_slots_zipf", T=16384, H=4096, I=1024, E=64, K=8,
                       renormalize=True, dtype="bf16", router="zipf", n_replicated=16),
        # the 60-expert layer with a shared-expert output added, and with the
        # routing weights applied on the expert input
        WorkloadConfig("qwen2_moe_shared_bf16", T=4096, H=2048, I=1408, E=60, K=4,
                       renormalize=False, dtype="bf16", router="gauss", shared_expert=True),
        WorkloadConfig("qwen2_moe_input_routing_bf16", T=4096, H=2048, I=1408, E=60, K=4,
                       renormalize=False, dtype="bf16", router="gauss", routing_on_input=True),
        # the 160-expert layer routed with 8 groups of 20 experts, 3 groups kept
        WorkloadConfig("deepseek_v2_grouped_bf16", T=8192, H=5120, I=1536, E=160, K=6,
                       renormalize=True, dtype="bf16", router="gauss_bias", bias_std=0.5,
                       num_expert_group=8, topk_group=3),
        # FP8 (E4M3) expert weights and activations on the two largest shapes
        WorkloadConfig("redundant_slots_zipf_fp8", T=16384, H=4096, I=1024, E=64, K=8,
                       renormalize=True, dtype="fp8", router="zipf", n_replicated=16),
        WorkloadConfig("deepseek_v2_fp8", T=8192, H=5120, I=1536, E=160, K=6,
                       renormalize=True, dtype="fp8", router="gauss_bias", bias_std=0.5),
    ]
}


def get_config(name: str, **overrides) -> WorkloadConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def small(name: str, T: int, H: Optional[int] = None, I: Optional[int] = None,
          **kw) -> WorkloadConfig:
    """A reduced copy of a named workload (same router and structure)."""
    cfg = CONFIGS[name]
    return cfg.replace(name=f"{name}_T{T}", T=T, H=H or cfg.H, I=I or cfg.I, **kw)
