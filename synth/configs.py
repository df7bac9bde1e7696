"""Shapes of the MoGE layer workloads (seeded synthetic inputs only).

Layer shape for the Pangu-Pro-sized cases: hidden 5120, 64 routed experts split
into 8 equal groups with one expert taken per group per token, and 4 always-on
shared experts (TechWalker, "Huawei releases Pangu Pro MoE", section 二 hardware
co-design; mokono.cn, "Pangu Pro MoE", 核心亮点 item 1).  The routed/shared
intermediate width 1344 is a synthetic choice: the pages do not print it.

Names:
  T tokens, d hidden, N routed experts, M groups, kp experts per group (K' in the
  pages), K = M*kp slots per token, inter = routed SwiGLU width,
  n_shared * shared_inter = I_s, the width of the concatenated shared SwiGLU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    N: int
    M: int
    kp: int
    inter: int
    n_shared: int
    shared_inter: int
    dtype: str            # "f32" or "bf16"
    w_std: float          # expert and shared weights ~ N(0, w_std)
    router_std: float     # router weight ~ N(0, router_std)
    x_std: float = 1.0
    zipf_s: float = 0.0   # >0: per-expert router bias -s*ln(e+1)
    seed: int = 0
    note: str = ""

    @property
    def G(self) -> int:
        return self.N // self.M

    @property
    def K(self) -> int:
        return self.M * self.kp

    @property
    def R(self) -> int:
        return self.T * self.K

    @property
    def I_s(self) -> int:
        return self.n_shared * self.shared_inter

    def with_T(self, T: int) -> "LayerConfig":
        return replace(self, T=T)


C0 = LayerConfig("C0-tiny-fp32", T=64, d=256, N=16, M=4, kp=1, inter=128,
                 n_shared=1, shared_inter=256, dtype="f32", w_std=0.02,
                 router_std=0.1,
                 note="tiny fp32 MoGE layer; the oracle finishes well under a second")
C1 = LayerConfig("C1-decode-T64", T=64, d=5120, N=64, M=8, kp=1, inter=1344,
                 n_shared=4, shared_inter=1344, dtype="bf16", w_std=0.02,
                 router_std=1.0 / math.sqrt(5120),
                 note="Pangu-Pro-shaped MoGE layer, decode batch of 64 tokens")
C2 = replace(C1, name="C2-decode-T456", T=456,
             note="same layer, large decode batch (456 tokens)")
C3 = replace(C1, name="C3-prefill-2x2048", T=4096,
             note="same layer, prefill of 2 sequences x 2048 tokens")
C4 = replace(C1, name="C4-skewed-T16384", T=16384, zipf_s=1.2,
             note="same layer, Zipf(1.2)-biased router, 16384 tokens")

CONFIGS = {"C0": C0, "C1": C1, "C2": C2, "C3": C3, "C4": C4}


def get(name: str) -> LayerConfig:
    return CONFIGS[name]
