"""Workload shapes for the 4-bit MoE prefill layer.

The A3B-class layer shapes (hidden 2048, 128 or 256 routed experts, top-8,
expert intermediate 768 or 512) stand in for the Qwen3.6-35B-A3B-class MoE
layers whose prefill the hipfire 0.4.3 benchmark page measures ("Qwen3.6-35B-A3B
prefill on the R9700" table, pp512 ... pp16384) and whose MoE prefill route is
the "symmetric IU4 MoE" route (40 layers, "Read this before comparing columns"
defaults table). The pages give no layer dimensions; these come from the
workload definition of this repository and are documented with the recipe.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens (prefill rows) per call
    H: int                 # hidden size
    E: int                 # routed experts
    k: int                 # experts per token
    I: int                 # routed expert intermediate size
    G: int                 # quantization group size along K
    quant: str             # "sym": w=(q-8)*scale ; "asym": w=q*scale+min
    shared_I: int = 0      # shared expert intermediate (0 = none)
    zipf_bias: bool = False  # router bias b[e] = 2*ln(1/(e+1))
    n_layers: int = 1      # >1: RMSNorm + residual stack
    chunk: int = 0         # rows per chunk for the stack (0 = T)
    seed: int = 0
    sweep_T: Tuple[int, ...] = field(default_factory=tuple)
    rms_eps: float = 1e-6

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_T(self, T: int) -> "MoEConfig":
        return replace(self, T=T)

    # Algorithmic work, counted without tile padding.
    def mfma_flops(self, T: int | None = None) -> float:
        """bf16 matrix flops of one layer: gate/up (4*H*I per pair) + down
        (2*H*I per pair), plus the shared expert on every token."""
        T = self.T if T is None else T
        return 6.0 * self.H * self.I * T * self.k + 6.0 * self.H * self.shared_I * T

    def gateup_flops(self, T: int | None = None) -> float:
        T = self.T if T is None else T
        return 4.0 * self.H * self.I * T * self.k

    def expert_bytes(self) -> int:
        """Packed bytes of one routed expert: nibbles + fp16 scales (+ mins)."""
        per = 2 if self.quant == "sym" else 4
        w = 3 * self.H * self.I // 2
        sc = (2 * self.I * (self.H // self.G) + self.H * (self.I // self.G)) * per
        return w + sc

    def shared_bytes(self) -> int:
        if not self.shared_I:
            return 0
        per = 2 if self.quant == "sym" else 4
        w = 3 * self.H * self.shared_I // 2
        sc = (2 * self.shared_I * (self.H // self.G) + self.H * (self.shared_I // self.G)) * per
        return w + sc + 4 * self.H


CONFIGS = {
    # Tiny layer: full brute-force checks finish instantly.
    "tiny": MoEConfig("tiny", T=64, H=256, E=8, k=2, I=128, G=32, quant="sym", seed=0),
    # A3B-shaped layer at a 512-row prefill chunk.
    "a3b_pp512": MoEConfig("a3b_pp512", T=512, H=2048, E=128, k=8, I=768, G=128,
                           quant="sym", seed=0),
    # Same layer at the 8192-row prefill chunk (compute-bound), plus the
    # weight-streaming sweep over the first 1/4/16 rows of the same tokens.
    "a3b_pp8192": MoEConfig("a3b_pp8192", T=8192, H=2048, E=128, k=8, I=768, G=128,
                            quant="sym", seed=0, sweep_T=(1, 4, 16)),
    # Skewed (Zipf-biased) routing with an always-on shared expert,
    # asymmetric int4 with group 32.
    "skew_shared": MoEConfig("skew_shared", T=4096, H=2048, E=256, k=8, I=512, G=32,
                             quant="asym", shared_I=512, zipf_bias=True, seed=0),
    # 40 skew_shared-shaped layers, each preceded by RMSNorm with a residual
    # add, over 16384 tokens in two 8192-row chunks.
    "stack40": MoEConfig("stack40", T=16384, H=2048, E=256, k=8, I=512, G=32,
                         quant="asym", shared_I=512, zipf_bias=True, n_layers=40,
                         chunk=8192, seed=0),
}

# Index order of the workload list the configs were defined from.
CONFIG_ORDER = ["tiny", "a3b_pp512", "a3b_pp8192", "skew_shared", "stack40"]


def get_config(name: str) -> MoEConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}")
