"""Shapes and storage formats of the five synthetic MoE-layer workloads.

Each workload is one MoE layer forward over T tokens. The dimensions follow the
config facts the pages print:

* dots3-note: hidden 5120, moe_intermediate 1536, 256 routed + 1 shared expert,
  top-8, sigmoid scoring, noaux_tc, norm_topk_prob, BF16/FP8
  ("dots3-note 架构深度解析" on mlqm.cn, parameter table «核心架构参数一览» and
  the «稀疏激活Top-8 路由» section).
* dots.llm1 lineage: top-6 of 128 routed + 2 shared, moe_intermediate 1408
  (Transformers "dots.llm1（Dots1）" article, model background list and the
  «MoE 路由与专家相关字段» table). The hidden size of that workload is 4096.
* Router groups (n_group, topk_group; default 1 and 1) and rms_norm_eps 1e-6
  come from the same article's field tables.

This module holds shapes only; it computes nothing of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int          # selects the RNG streams of the workload
    T: int               # tokens (batch * sequence, flattened)
    H: int               # hidden size
    E: int               # routed experts
    S: int               # shared experts
    k: int               # experts per token
    I: int               # routed expert intermediate size
    Is: int              # shared expert intermediate size
    act: str             # storage type of x, router weight and output: "f32" | "bf16"
    expert: str          # storage type of expert weights: "f32" | "bf16" | "fp8"
    bias_kind: str = "uniform"   # "uniform": U(-0.01, 0.01); "zipf": skewed popularity
    zipf_s: float = 1.2
    zipf_lambda: float = 0.10
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 1.0
    n_group: int = 1             # expert groups of the router (1: no grouping)
    topk_group: int = 1          # groups a token may choose from
    rms_norm_eps: float = 1e-6   # decoder-block RMSNorm epsilon
    weight_std: float = 0.02
    bias_half_width: float = 0.01

    @property
    def rows(self) -> int:
        """Routed (token, slot) pairs."""
        return self.T * self.k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    def flops(self) -> float:
        """Matmul flops of one layer forward: router + routed + shared SwiGLU."""
        return float(self.T) * (2.0 * self.H * self.E
                                + 6.0 * self.H * (self.k * self.I + self.S * self.Is))


CONFIGS = {
    0: MoEConfig("tiny_fp32", 0, T=64, H=512, E=32, S=1, k=4, I=128, Is=128,
                 act="f32", expert="f32"),
    1: MoEConfig("dots3_decode_T256_bf16", 1, T=256, H=5120, E=256, S=1, k=8,
                 I=1536, Is=1536, act="bf16", expert="bf16"),
    2: MoEConfig("dots3_prefill_T16384_bf16", 2, T=16384, H=5120, E=256, S=1, k=8,
                 I=1536, Is=1536, act="bf16", expert="bf16"),
    3: MoEConfig("dotsllm1_skewed_T8192_bf16", 3, T=8192, H=4096, E=128, S=2, k=6,
                 I=1408, Is=1408, act="bf16", expert="bf16", bias_kind="zipf"),
    4: MoEConfig("dots3_fp8_T4096", 4, T=4096, H=5120, E=256, S=1, k=8,
                 I=1536, Is=1536, act="bf16", expert="fp8"),
}


def config(cfg_id: int, **overrides) -> MoEConfig:
    c = CONFIGS[cfg_id]
    return c.with_(**overrides) if overrides else c
