"""The five seeded synthetic workloads of the DeepSeekMoE layer forward.

Shapes follow the DeepSeek-V3 technical-report summary (1 shared + 256 routed
experts, 8 active; section "核心概念") for the V3-shaped cases, and smaller
tiny/mid cases for parity.  Distributions: tokens u ~ N(0,1); centroids
e_i ~ N(0, 1/d); expert weights ~ N(0, 1/fan_in) with fan_in = d for the
gate/up projections and I for the down projection.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    tokens: int        # T
    hidden: int        # d
    n_routed: int      # N_r
    top_k: int         # K_r
    n_shared: int      # N_s
    inter: int         # I (intermediate width of every expert's SwiGLU FFN)
    dtype: str         # "f32" | "bf16" | "fp8"
    bias: str          # "zero" | "uniform0.01" | "normal_var0.01"
    zipf: bool = False  # centroid norms scaled for Zipf(1.1)-like popularity
    steps: int = 1      # route + forward + bias-update steps in the workload
    gamma: float = 0.001
    seed: int = 0

    @property
    def total_assignments(self) -> int:
        return self.tokens * self.top_k

    def flops_per_token(self) -> int:
        """Algorithmic flops per token: router logits + (K_r + N_s) SwiGLU FFNs."""
        return 2 * self.n_routed * self.hidden + (self.top_k + self.n_shared) * 6 * self.hidden * self.inter

    def with_tokens(self, t: int) -> "LayerConfig":
        d = dict(self.__dict__)
        d["tokens"] = t
        return LayerConfig(**d)


CONFIGS = {
    0: LayerConfig(0, "tiny-f32", 64, 128, 16, 4, 1, 64, "f32", "zero", steps=1),
    1: LayerConfig(1, "mid-bf16", 4096, 2048, 64, 6, 2, 1408, "bf16", "uniform0.01"),
    2: LayerConfig(2, "v3-decode-bf16", 256, 7168, 256, 8, 1, 2048, "bf16", "normal_var0.01"),
    3: LayerConfig(3, "v3-prefill-bf16-zipf", 16384, 7168, 256, 8, 1, 2048, "bf16", "zero",
                   zipf=True, steps=20),
    4: LayerConfig(4, "v3-prefill-fp8", 8192, 7168, 256, 8, 1, 2048, "fp8", "normal_var0.01"),
}


def get_config(cid: int) -> LayerConfig:
    return CONFIGS[cid]
