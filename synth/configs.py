"""Named workload shapes of the DeepSeekMoE layer forward pass.

The five named workloads follow the shapes the pages give for DeepSeek-V3
(256 routed experts of intermediate width 2048, top-8, one shared expert,
hidden 7168; "DeepSeekMoE" explainer, sections 1 and 2.1) and for the 2024
DeepSeekMoE layout (2 shared + 64 routed experts, 2+6 active, gates not
renormalised; course notes, sections 3 and 4). Value distributions are the
synthetic recipe of this library: x ~ N(0, x_std^2), weights ~ N(0, w_std^2),
bias ~ U(-bias_range, bias_range).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

SCORE_SIGMOID = "sigmoid"
SCORE_SOFTMAX = "softmax"
NORM_SELECTED = "selected"
NORM_NONE = "none"


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens in the batch
    d: int                 # hidden size
    E: int                 # routed experts
    K: int                 # experts selected per token
    I: int                 # routed expert intermediate width
    S: int                 # shared experts
    Is: int                # shared expert intermediate width (each)
    score: str = SCORE_SIGMOID
    norm: str = NORM_SELECTED
    act_dtype: str = "bf16"      # "f32" | "bf16"
    weight_dtype: str = "bf16"   # "f32" | "bf16" | "fp8"
    out_dtype: str = "f32"       # layer output y: "f32" | "bf16"
    # gate-weighted routed rows out_slots: "f32" | "bf16". The full-size bf16
    # workloads hold them in bf16 (half the bytes the down GEMM writes and the
    # combine reads); reduced shapes keep the library default, fp32, unless
    # they ask (scaled_config)
    slot_dtype: str = "f32"
    bias_range: Optional[float] = None   # None -> no bias tensor
    x_std: float = 1.0
    w_std: float = 0.02
    seed: int = 20260100
    # Zipf-popularity router construction (stress workload)
    zipf_s: Optional[float] = None
    zipf_A: Optional[float] = None
    batches: int = 1
    gamma: float = 1e-3
    # node-limited routing ("DeepSeekMoE" explainer, section 2.3): experts in
    # n_groups groups of E/n_groups, topk_groups groups kept per token (0 = off)
    n_groups: int = 0
    topk_groups: int = 0
    # fp8 weight scales: "row" = one fp32 scale per output row (bf16
    # activations); "block" = one per 128 x 128 block, with the activations
    # quantised to fp8 in 1 x 128 tiles on the fly ("DeepSeekMoE" explainer,
    # section 4.3)
    fp8_scaling: str = "row"
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def tk(self) -> int:
        return self.T * self.K

    def flops(self) -> float:
        """Algorithmic FLOPs of one layer call: router GEMM, routed SwiGLU
        experts over the T*K selected (token, expert) pairs, shared experts."""
        router = 2.0 * self.T * self.d * self.E
        routed = 6.0 * self.d * self.I * self.T * self.K
        shared = 6.0 * self.d * self.Is * self.S * self.T
        return router + routed + shared

    def weight_bytes_per_expert(self) -> int:
        wb = {"f32": 4, "bf16": 2, "fp8": 1}[self.weight_dtype]
        b = 3 * self.d * self.I * wb
        if self.weight_dtype == "fp8":
            b += 4 * (3 * (self.I // 128) * (self.d // 128) if self.fp8_scaling == "block"
                      else 2 * self.I + self.d)
        return b

    def shared_weight_bytes(self) -> int:
        wb = {"f32": 4, "bf16": 2, "fp8": 1}[self.weight_dtype]
        b = 3 * self.d * self.Is * self.S * wb
        if self.weight_dtype == "fp8":
            b += 4 * (3 * (self.Is * self.S // 128) * (self.d // 128) if self.fp8_scaling == "block"
                      else 2 * self.Is * self.S + self.d)
        return b

    def act_bytes(self) -> int:
        return {"f32": 4, "bf16": 2}[self.act_dtype]


_BASE = 20260100

CONFIGS = {
    "tiny_f32": MoEConfig(
        name="tiny_f32", T=64, d=128, E=16, K=2, I=64, S=1, Is=64,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="f32", weight_dtype="f32",
        bias_range=0.1, x_std=0.02, w_std=0.02, seed=_BASE + 1,
        description="Tiny fp32 layer: 16 routed + 1 shared expert, sigmoid, top-2, biased selection",
    ),
    "dsmoe2024_bf16": MoEConfig(
        name="dsmoe2024_bf16", T=4096, d=2048, E=64, K=6, I=1408, S=2, Is=1408,
        score=SCORE_SOFTMAX, norm=NORM_NONE, act_dtype="bf16", weight_dtype="bf16",
        slot_dtype="bf16", bias_range=None, x_std=1.0, w_std=0.02, seed=_BASE + 2,
        description="DeepSeekMoE-2024 layout: 64 routed + 2 shared, softmax, top-6, no renormalisation",
    ),
    "v3_prefill_bf16": MoEConfig(
        name="v3_prefill_bf16", T=8192, d=7168, E=256, K=8, I=2048, S=1, Is=2048,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="bf16", weight_dtype="bf16",
        slot_dtype="bf16", bias_range=0.05, x_std=1.0, w_std=0.02, seed=_BASE + 3,
        description="V3-shape prefill: 256 routed + 1 shared, sigmoid, top-8 on score+bias",
    ),
    "v3_decode_fp8": MoEConfig(
        name="v3_decode_fp8", T=64, d=7168, E=256, K=8, I=2048, S=1, Is=2048,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="bf16", weight_dtype="fp8",
        bias_range=0.05, x_std=1.0, w_std=0.02, seed=_BASE + 4,
        description="V3-shape decode: fp8-e4m3 expert weights with per-output-row fp32 scales",
    ),
    "zipf_stress_bf16": MoEConfig(
        name="zipf_stress_bf16", T=32768, d=7168, E=256, K=8, I=2048, S=1, Is=2048,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="bf16", weight_dtype="bf16",
        slot_dtype="bf16", bias_range=None, x_std=1.0, w_std=0.02, seed=_BASE + 5,
        zipf_s=1.1, zipf_A=2.3828, batches=20, gamma=1e-3,   # A: oracle/calibrate_zipf.py
        description="Zipf(1.1) expert popularity (hottest ~10x mean load), 20 batches + bias update",
    ),
    "v3_grouped_bf16": MoEConfig(
        name="v3_grouped_bf16", T=8192, d=7168, E=256, K=8, I=2048, S=1, Is=2048,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="bf16", weight_dtype="bf16",
        slot_dtype="bf16", bias_range=0.05, x_std=1.0, w_std=0.02, seed=_BASE + 6,
        n_groups=8, topk_groups=4,
        description="V3-shape prefill with node-limited routing: 8 groups of 32 experts, top-4 groups",
    ),
    "v3_prefill_fp8b": MoEConfig(
        name="v3_prefill_fp8b", T=8192, d=7168, E=256, K=8, I=2048, S=1, Is=2048,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="bf16", weight_dtype="fp8",
        fp8_scaling="block", bias_range=0.05, x_std=1.0, w_std=0.02, seed=_BASE + 7,
        description="V3-shape prefill in fine-grained fp8: 128x128 weight blocks, 1x128 activation tiles",
    ),
    "v3_ep8_shard_bf16": MoEConfig(
        name="v3_ep8_shard_bf16", T=8192, d=7168, E=32, K=8, I=2048, S=1, Is=2048,
        score=SCORE_SIGMOID, norm=NORM_SELECTED, act_dtype="bf16", weight_dtype="bf16",
        slot_dtype="bf16", bias_range=0.05, x_std=1.0, w_std=0.02, seed=_BASE + 8,
        description="One GPU's share of the V3 prefill layer under 8-way expert parallelism: "
                    "32 local experts receiving 8 x 8192 x 8 / 256 = 2048 routed rows each, "
                    "the shared expert on the 8192 local tokens",
    ),
}


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]


def scaled_config(base_name: str, **overrides) -> MoEConfig:
    """A named workload with some fields replaced (reduced sizes for tests).
    The slot rows go back to the library default (fp32) unless slot_dtype is
    among the overrides: with one routed slot and no shared expert a single
    bf16 slot row can be the whole output, and its rounding alone then
    approaches the 2e-2 x RMS bar."""
    base = CONFIGS[base_name]
    new_name = overrides.pop("name", base.name + "_scaled")
    overrides.setdefault("slot_dtype", "f32")
    return dataclasses.replace(base, name=new_name, **overrides)
