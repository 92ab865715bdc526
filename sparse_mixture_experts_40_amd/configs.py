"""The five synthetic MoE-block workloads.

Shapes come from the two model families on the pages: the 128-expert / top-8 /
I=1536 / H=4096 configuration ([MOE-128x8] "MoE架构深度解析：128专家与8激活的智能路由",
config JSON) and the Mixtral 8-choose-2 block ([QWEN3-READ] "大模型-qwen3 MoE
详细解读", §三 Mixtral difference: no renormalisation).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # hidden_size
    E: int          # num_experts
    k: int          # num_experts_per_tok
    I: int          # moe_intermediate_size
    norm: bool      # norm_topk_prob
    dtype: str      # "f32" or "bf16"
    zipf_s: float = 0.0   # > 0: per-expert logit bias log(Zipf(s)) (skewed loads)
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "MoEConfig":
        return MoEConfig(self.name, T, self.H, self.E, self.k, self.I, self.norm, self.dtype,
                         self.zipf_s, self.seed)


TINY_F32 = MoEConfig("tiny_f32", T=64, H=128, E=8, k=2, I=256, norm=True, dtype="f32")
MIXTRAL_BF16 = MoEConfig("mixtral_bf16", T=4096, H=4096, E=8, k=2, I=14336, norm=False,
                         dtype="bf16")
FINEGRAINED_BF16 = MoEConfig("finegrained_bf16", T=8192, H=2048, E=64, k=8, I=1024, norm=True,
                             dtype="bf16")
PREFILL128_BF16 = MoEConfig("prefill128_bf16", T=16384, H=4096, E=128, k=8, I=1536, norm=True,
                            dtype="bf16")
DECODE128_BF16 = MoEConfig("decode128_bf16", T=64, H=4096, E=128, k=8, I=1536, norm=True,
                           dtype="bf16", zipf_s=1.2)

WORKLOADS = {c.name: c for c in (TINY_F32, MIXTRAL_BF16, FINEGRAINED_BF16, PREFILL128_BF16,
                                 DECODE128_BF16)}
