"""The five layer shapes the MoE-layer forward is exercised and measured on.

Shapes come from the pages: Qwen3-30B-A3B (H 2048, E 128, k 8, F 768) and
DeepSeek-V3 (H 7168, E 256, k 8, F 2048, 8 groups, best 4) from [MoE]
"Shapes, sourced"; GLM-5.3-Flash (H 4096, 288 experts, top 8) from [Router]
§1.1; DeepSeek-V4-Flash (H 4096, 256 experts, k 6, 2 x 2048 gate/up) from
[MegaMoE] §1.1.  GLM's F (2304) and the value distributions are not printed
on the pages; they are stated with the configurations of this project.

Selection-bias spread: N(0, 0.1) where it is given (GLM).  For the two
DeepSeek shapes no spread is given; N(0, 0.01) is used because the pages'
workloads for them route near-uniformly (about 222 of 256 experts touched by
64 tokens in the [MoE] DeepSeek-V3 trace; random routing with every expert
getting about the same number of tokens in [MegaMoE] §1.3), while N(0, 0.1)
with saturated sigmoid scores concentrates the choice on half the experts.
"""

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int
    E: int
    k: int
    F: int
    scoring: str                  # "softmax" | "sigmoid"
    has_bias: bool
    wformat: str                  # "bf16" | "fp8" | "mxfp4"
    Ts: Tuple[int, ...]
    n_group: int = 1
    topk_group: int = 1
    renormalize: bool = True
    routed_scale: float = 1.0
    x_std: float = 1.0
    gate_std: float = 0.02
    w_std: float = 0.02
    bias_std: float = 0.1
    seed: int = 0
    description: str = field(default="", compare=False)

    def expert_bytes(self):
        """Stored bytes of one expert (w13 + w2, scales included)."""
        H, F = self.H, self.F
        if self.wformat == "bf16":
            return 6 * H * F
        if self.wformat == "fp8":
            cd = lambda a: -(-a // 128)
            return 3 * H * F + 4 * (cd(2 * F) * cd(H) + cd(H) * cd(F))
        if self.wformat == "mxfp4":
            return 3 * H * F // 2 + (2 * F * H + H * F) // 32
        raise ValueError(self.wformat)


CONFIGS = {
    "toy": LayerConfig(
        "toy", H=256, E=8, k=2, F=128, scoring="softmax", has_bias=False,
        wformat="bf16", Ts=(16,), seed=0,
        description="toy MoE layer, softmax top-2 + renormalise"),
    "qwen3": LayerConfig(
        "qwen3", H=2048, E=128, k=8, F=768, scoring="softmax", has_bias=False,
        wformat="bf16", Ts=(1, 64, 4096),
        description="Qwen3-30B-A3B-shaped layer, softmax top-8, bf16 experts"),
    "glm": LayerConfig(
        "glm", H=4096, E=288, k=8, F=2304, scoring="sigmoid", has_bias=True,
        wformat="bf16", Ts=(1, 8, 512),
        description="GLM-5.3-Flash-shaped layer, sigmoid + fp32 bias top-8, bf16 experts"),
    "dsv3": LayerConfig(
        "dsv3", H=7168, E=256, k=8, F=2048, scoring="sigmoid", has_bias=True,
        wformat="fp8", Ts=(1, 256, 2048), n_group=8, topk_group=4,
        routed_scale=2.5, bias_std=0.01,
        description="DeepSeek-V3-shaped layer, grouped sigmoid + bias top-8, fp8 128x128 experts"),
    "dsv4": LayerConfig(
        "dsv4", H=4096, E=256, k=6, F=2048, scoring="sigmoid", has_bias=True,
        wformat="mxfp4", Ts=(512, 8192), bias_std=0.01,
        description="DeepSeek-V4-Flash-shaped layer, sigmoid + bias top-6, MXFP4 x fp8"),
}


def get_config(name, **overrides):
    """A named configuration, optionally with fields replaced (e.g. a smaller
    E or H for a test that must run in seconds)."""
    base = CONFIGS[name]
    if not overrides:
        return base
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(overrides)
    return LayerConfig(**d)
