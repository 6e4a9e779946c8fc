"""Named MoE-layer workloads: shapes, routing hyper-parameters, precision recipes.

The hyper-parameter names follow the DeepSeek-V3 configuration keys that the
Kimi-K2-Thinking-NVFP4 walk-through (pwwt.cn, section 3 "MoE routing") uses:
num_experts_per_tok, topk_method "noaux_tc", n_group, topk_group,
norm_topk_prob, routed_scaling_factor.  The V4-Pro overview (lzwjava.github.io,
"architecture") adds the sqrtsoftplus score function and route_scale 2.5; the
2.8T open-weights articles (ruibaoantu.com, "expert layer" and "quantisation")
give 896 experts, top-16, 2 shared experts, MXFP4 weights and MXFP8
activations.

This module only describes workloads.  It computes nothing of the layer.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

# Precision recipes.  Numbers match the moe_recipe_t enum of include/moe.h.
RECIPE_F32 = 0          # x, experts, shared, out: fp32
RECIPE_BF16 = 1         # x, experts, shared, out: bf16
RECIPE_FP8_B128 = 2     # experts fp8 e4m3fn + fp32 128x128 block scales; activations fp8 per (row,128); shared bf16
RECIPE_MXFP4 = 3        # experts MXFP4 (e2m1 + E8M0 per 32); activations MXFP8 (e4m3fn + E8M0 per 32); shared bf16
RECIPE_NVFP4 = 4        # experts and their activations NVFP4 (e2m1 + e4m3 scale per 16); shared bf16

RECIPE_NAMES = {RECIPE_F32: "f32", RECIPE_BF16: "bf16", RECIPE_FP8_B128: "fp8_b128",
                RECIPE_MXFP4: "mxfp4_mxfp8", RECIPE_NVFP4: "nvfp4"}

SCORE_SIGMOID = 0
SCORE_SQRTSOFTPLUS = 1


@dataclass(frozen=True)
class MoEConfig:
    name: str
    num_tokens: int          # T
    hidden: int              # H
    num_experts: int         # E (routed)
    top_k: int               # k
    intermediate: int        # I of one routed expert
    num_shared: int          # number of always-on shared experts
    shared_intermediate: int  # I of one shared expert
    n_group: int = 1
    topk_group: int = 1
    score_func: int = SCORE_SIGMOID
    norm_topk_prob: bool = True
    routed_scaling_factor: float = 2.827
    recipe: int = RECIPE_BF16
    swiglu_limit: float = 0.0   # > 0: gate clamped to <= limit, up to [-limit, limit] before SiLU(g)*u
    # --- synthetic-input recipe (not layer hyper-parameters) ---
    seed: int = 0
    gate_std: float = 0.02
    expert_std: float = 0.02
    bias_kind: str = "normal"     # "normal" | "uniform" | "zipf"
    bias_param: float = 0.01      # std (normal) or half-width (uniform) or Zipf exponent
    description: str = ""

    @property
    def pairs(self) -> int:
        return self.num_tokens * self.top_k

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  c1 is small enough for the oracle to finish in seconds;
# c2..c5 are the full single-GPU layer shapes.
TINY_F32 = MoEConfig(
    name="tiny_fp32", num_tokens=64, hidden=256, num_experts=16, top_k=4,
    intermediate=128, num_shared=1, shared_intermediate=128,
    n_group=1, topk_group=1, score_func=SCORE_SIGMOID, routed_scaling_factor=2.827,
    recipe=RECIPE_F32, gate_std=1.0 / 16.0, bias_kind="uniform", bias_param=0.1,
    description="T=64 H=256 E=16 k=4 I=128, fp32, sigmoid, n_group=1, scale 2.827")

DECODE_BF16 = MoEConfig(
    name="decode_bf16", num_tokens=128, hidden=7168, num_experts=384, top_k=8,
    intermediate=2048, num_shared=1, shared_intermediate=2048,
    n_group=1, topk_group=1, score_func=SCORE_SIGMOID, routed_scaling_factor=2.827,
    recipe=RECIPE_BF16, bias_kind="normal", bias_param=0.01,
    description="T=128 H=7168 E=384 k=8 I=2048, bf16, sigmoid, n_group=1, scale 2.827")

PREFILL_BF16_GROUPED = MoEConfig(
    name="prefill_bf16_grouped", num_tokens=8192, hidden=7168, num_experts=256, top_k=8,
    intermediate=2048, num_shared=1, shared_intermediate=2048,
    n_group=8, topk_group=4, score_func=SCORE_SIGMOID, routed_scaling_factor=2.5,
    recipe=RECIPE_BF16, bias_kind="normal", bias_param=0.01,
    description="T=8192 H=7168 E=256 k=8 I=2048, bf16, sigmoid, n_group=8 topk_group=4, scale 2.5")

FINEGRAINED_MXFP4 = MoEConfig(
    name="finegrained_mxfp4", num_tokens=4096, hidden=7168, num_experts=896, top_k=16,
    intermediate=1024, num_shared=2, shared_intermediate=1024,
    n_group=1, topk_group=1, score_func=SCORE_SIGMOID, routed_scaling_factor=2.827,
    recipe=RECIPE_MXFP4, bias_kind="normal", bias_param=0.01,
    description="T=4096 H=7168 E=896 k=16 I=1024 x2 shared, MXFP4 weights x MXFP8 activations")

SKEWED_FP8 = MoEConfig(
    name="skewed_fp8", num_tokens=16384, hidden=7168, num_experts=384, top_k=6,
    intermediate=2048, num_shared=1, shared_intermediate=2048,
    n_group=1, topk_group=1, score_func=SCORE_SQRTSOFTPLUS, routed_scaling_factor=2.5,
    recipe=RECIPE_FP8_B128, bias_kind="zipf", bias_param=1.1,
    description="T=16384 H=7168 E=384 k=6 I=2048, fp8 128x128 blocks, sqrtsoftplus, Zipf(1.1) load")

FULL_CONFIGS = [TINY_F32, DECODE_BF16, PREFILL_BF16_GROUPED, FINEGRAINED_MXFP4, SKEWED_FP8]

# Small variants that keep each structure at a size the oracle finishes in
# well under a second (several tiles along every GEMM dimension, ragged tails).
MINI_GROUPED_BF16 = MoEConfig(
    name="mini_grouped_bf16", num_tokens=200, hidden=384, num_experts=32, top_k=6,
    intermediate=256, num_shared=1, shared_intermediate=256, n_group=4, topk_group=2,
    routed_scaling_factor=2.5, recipe=RECIPE_BF16, gate_std=1.0 / 16.0,
    description="grouped top-k mini (E=32, 4 groups keep 2)")

MINI_DECODE_BF16 = MoEConfig(
    name="mini_decode_bf16", num_tokens=5, hidden=512, num_experts=64, top_k=8,
    intermediate=384, num_shared=1, shared_intermediate=256,
    recipe=RECIPE_BF16, gate_std=1.0 / 16.0, description="decode-shaped mini, few tokens")

MINI_MXFP4 = MoEConfig(
    name="mini_mxfp4", num_tokens=160, hidden=512, num_experts=32, top_k=8,
    intermediate=256, num_shared=2, shared_intermediate=128,
    recipe=RECIPE_MXFP4, gate_std=1.0 / 16.0, description="MXFP4 x MXFP8 mini, 2 shared")

MINI_FP8 = MoEConfig(
    name="mini_fp8", num_tokens=300, hidden=384, num_experts=24, top_k=6,
    intermediate=256, num_shared=1, shared_intermediate=256,
    score_func=SCORE_SQRTSOFTPLUS, routed_scaling_factor=2.5,
    recipe=RECIPE_FP8_B128, gate_std=1.0 / 16.0, bias_kind="zipf", bias_param=1.1,
    description="fp8 128-block mini with sqrtsoftplus and Zipf load")

MINI_F32 = MoEConfig(
    name="mini_f32", num_tokens=97, hidden=192, num_experts=12, top_k=3,
    intermediate=96, num_shared=1, shared_intermediate=64,
    recipe=RECIPE_F32, gate_std=1.0 / 16.0, bias_kind="uniform", bias_param=0.1,
    description="fp32 mini with ragged sizes")

MINI_PREFILL_BF16 = MoEConfig(
    name="mini_prefill_bf16", num_tokens=512, hidden=384, num_experts=8, top_k=4,
    intermediate=256, num_shared=1, shared_intermediate=256, n_group=2, topk_group=2,
    routed_scaling_factor=2.5, recipe=RECIPE_BF16, gate_std=1.0 / 16.0,
    description="prefill-shaped bf16 mini: 256-row tiles, ragged experts, partial column tile")

MINI_PREFILL_FP8 = MoEConfig(
    name="mini_prefill_fp8", num_tokens=512, hidden=512, num_experts=8, top_k=2,
    intermediate=256, num_shared=1, shared_intermediate=128,
    score_func=SCORE_SQRTSOFTPLUS, routed_scaling_factor=2.5, recipe=RECIPE_FP8_B128,
    gate_std=1.0 / 16.0, description="prefill-shaped fp8 mini: 128-row tiles")

MINI_MXFP4_WIDE = MoEConfig(
    name="mini_mxfp4_wide", num_tokens=560, hidden=512, num_experts=16, top_k=4,
    intermediate=256, num_shared=1, shared_intermediate=128,
    recipe=RECIPE_MXFP4, gate_std=1.0 / 16.0,
    description="MXFP4 mini with about 140 rows per expert: two or three ragged row tiles per expert")

MINI_MIXED_BF16 = MoEConfig(
    name="mini_mixed_bf16", num_tokens=300, hidden=384, num_experts=24, top_k=6,
    intermediate=256, num_shared=1, shared_intermediate=256,
    routed_scaling_factor=2.5, recipe=RECIPE_BF16, gate_std=1.0 / 16.0, bias_kind="zipf", bias_param=1.1,
    description="bf16 mini with a Zipf load: empty experts, 128-row register-streaming tiles and "
                "256-row LDS tiles in one call, partial column tiles")

MINI_NVFP4 = MoEConfig(
    name="mini_nvfp4", num_tokens=160, hidden=512, num_experts=32, top_k=8,
    intermediate=256, num_shared=1, shared_intermediate=128,
    recipe=RECIPE_NVFP4, gate_std=1.0 / 16.0, description="NVFP4 mini (32-to-64-row tiles)")

MINI_NVFP4_WIDE = MoEConfig(
    name="mini_nvfp4_wide", num_tokens=560, hidden=512, num_experts=16, top_k=4,
    intermediate=256, num_shared=1, shared_intermediate=128,
    recipe=RECIPE_NVFP4, gate_std=1.0 / 16.0,
    description="NVFP4 mini with about 140 rows per expert: 128-row tiles")

MINI_SKEWED_FP8 = MoEConfig(
    name="mini_skewed_fp8", num_tokens=1200, hidden=384, num_experts=12, top_k=2,
    intermediate=256, num_shared=1, shared_intermediate=128,
    score_func=SCORE_SQRTSOFTPLUS, routed_scaling_factor=2.5, recipe=RECIPE_FP8_B128,
    gate_std=1.0 / 16.0, bias_kind="zipf", bias_param=1.1,
    description="fp8 mini averaging 200 rows per expert with a Zipf load: heavy experts of several "
                "192-row tiles, run in groups of row tiles")

MINI_CONFIGS = [MINI_GROUPED_BF16, MINI_DECODE_BF16, MINI_MXFP4, MINI_FP8, MINI_F32, MINI_PREFILL_BF16,
                MINI_PREFILL_FP8, MINI_MXFP4_WIDE, MINI_MIXED_BF16, MINI_NVFP4, MINI_NVFP4_WIDE, MINI_SKEWED_FP8]

# NVFP4 (walk-through section 4): the decode shape of the Kimi-K2-Thinking-NVFP4 /
# DeepSeek-V3 layer with NVFP4 routed experts; not one of the five workloads above.
DECODE_NVFP4 = DECODE_BF16.replace(
    name="decode_nvfp4", recipe=RECIPE_NVFP4,
    description="T=128 H=7168 E=384 k=8 I=2048, NVFP4 routed experts and activations, bf16 shared expert")

NEXT_CONFIGS = [DECODE_NVFP4]

BY_NAME = {c.name: c for c in FULL_CONFIGS + MINI_CONFIGS + NEXT_CONFIGS}


def get(name: str) -> MoEConfig:
    return BY_NAME[name]
