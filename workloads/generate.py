"""Seeded synthetic inputs for one MoE layer, in the storage formats the layer reads.

Every tensor draws from its own torch.Generator, seeded from
(config seed, config name, tensor id, expert id), so that any expert can be
regenerated alone.  Values are drawn in fp32 and rounded to the storage format
(bf16 round-to-nearest-even by torch's cast; fp8 e4m3fn by torch's cast after
a 128x128 amax/448 block scale; MXFP4 by the e2m1 encoder below).

Encoding weights is input preparation, as the V4-Pro overview's convert.py
step is (lzwjava.github.io, "convert.py"): this module holds no step of the
layer's forward pass (no scoring, selection, permutation, activation
quantisation, matrix product or combine).

Reading of "N(0, v)" in the workload descriptions: N(0, 1/256) is a variance
(sigma = 1/16, unit-variance logits at H = 256); N(0, 0.02) and N(0, 0.01) are
standard deviations (the initializer-range convention).
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

from . import configs as C

# e2m1 magnitudes by code (sign is bit 3): OCP Microscaling Formats v1.0, table of FP4 E2M1.
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
# At each midpoint a tie goes to the neighbour with the even code.
_E2M1_TIE_UP = (False, True, False, True, False, True, False)
E4M3_MAX = 448.0
E2M1_MAX = 6.0

TENSOR_IDS = {"x": 1, "gate_w": 2, "bias": 3, "w13": 4, "w2": 5, "shared_w13": 6, "shared_w2": 7,
              "zipf_perm": 8, "norm_w": 9}

# post_attention_layernorm epsilon of the residual form (not stated by the pages;
# the usual DeepSeek config value)
RMS_EPS = 1e-6


def tensor_seed(cfg: C.MoEConfig, tensor: str, expert: int = 0) -> int:
    ss = np.random.SeedSequence([cfg.seed, zlib.crc32(cfg.name.encode()), TENSOR_IDS[tensor], expert])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(cfg, tensor, expert, device):
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(cfg, tensor, expert))
    return g


def normal(cfg, tensor, expert, shape, std, device="cpu"):
    g = _gen(cfg, tensor, expert, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


# ---------------------------------------------------------------- weight encoders
def encode_fp8_block128(w: torch.Tensor):
    """fp32 [R, K] -> (e4m3fn codes uint8 [R, K], fp32 scales [R/128, K/128]); s = amax/448."""
    R, K = w.shape
    assert R % 128 == 0 and K % 128 == 0
    blk = w.reshape(R // 128, 128, K // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = q.reshape(R, K).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.contiguous()


def encode_e2m1(v: torch.Tensor) -> torch.Tensor:
    """Round |v| <= 6 to the e2m1 grid (ties to even code); returns 4-bit codes as uint8."""
    a = v.abs().clamp(max=E2M1_MAX)
    code = torch.zeros_like(a, dtype=torch.uint8)
    for mid, up in zip(_E2M1_MIDPOINTS, _E2M1_TIE_UP):
        code += (a >= mid if up else a > mid).to(torch.uint8)
    sign = ((v < 0) & (code > 0)).to(torch.uint8) << 3
    return code | sign


def encode_nvfp4(w: torch.Tensor):
    """fp32 [R, K] -> (packed e2m1 uint8 [R, K/2] low nibble = even k, e4m3fn scale codes uint8 [R, K/16]).

    Per 16 consecutive values: scale = e4m3(amax / 6) (1 when that rounds to 0),
    codes = e2m1(v / scale)."""
    R, K = w.shape
    assert K % 16 == 0
    blk = w.reshape(R, K // 16, 16)
    amax = blk.abs().amax(dim=2)
    sc = (amax / E2M1_MAX).to(torch.float8_e4m3fn)
    s = sc.to(torch.float32)
    one = torch.ones_like(s)
    sc = torch.where(s > 0, sc.view(torch.uint8), one.to(torch.float8_e4m3fn).view(torch.uint8))
    s = torch.where(s > 0, s, one)
    codes = encode_e2m1(blk / s[:, :, None]).reshape(R, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.contiguous(), sc.contiguous()


def encode_mxfp4(w: torch.Tensor):
    """fp32 [R, K] -> (packed e2m1 uint8 [R, K/2] low nibble = even k, E8M0 uint8 [R, K/32]).

    Block exponent e = the smallest integer with amax <= 6 * 2^e (no element clips);
    an all-zero block takes e = 0.
    """
    R, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(R, K // 32, 32)
    amax = blk.abs().amax(dim=2)
    e = torch.zeros_like(amax, dtype=torch.int32)
    nz = amax > 0
    # initial guess from frexp, then fix up with exact power-of-two comparisons
    m, ex = torch.frexp(torch.where(nz, amax / E2M1_MAX, torch.ones_like(amax)))
    e = torch.where(nz, ex.to(torch.int32), e)               # amax/6 < 2^ex
    for _ in range(2):
        smaller_ok = nz & (amax <= E2M1_MAX * torch.ldexp(torch.ones_like(amax), (e - 1).float()))
        e = torch.where(smaller_ok, e - 1, e)
    e = e.clamp(-127, 127)
    scaled = blk * torch.ldexp(torch.ones_like(amax), (-e).float())[:, :, None]
    codes = encode_e2m1(scaled).reshape(R, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


# ---------------------------------------------------------------- bias for skewed load
def zipf_target(cfg: C.MoEConfig):
    """The seeded expert ranking (1 = most loaded) and the target pick probabilities
    q_e = k * p_rank(e), p_r proportional to r^-s, water-filled under a cap of 0.995
    so that sum q_e = k (float64 tensors [E])."""
    E, k, s = cfg.num_experts, cfg.top_k, cfg.bias_param
    g = torch.Generator().manual_seed(tensor_seed(cfg, "zipf_perm"))
    perm = torch.randperm(E, generator=g)
    rank = torch.empty(E, dtype=torch.float64)
    rank[perm] = torch.arange(1, E + 1, dtype=torch.float64)
    p = rank ** (-s)
    p = p / p.sum()
    cap = 0.995
    q = k * p
    fixed = torch.zeros(E, dtype=torch.bool)
    for _ in range(E):
        over = (q > cap) & ~fixed
        if not bool(over.any()):
            break
        fixed |= over
        q[fixed] = cap
        rest = k - cap * fixed.sum()
        free = ~fixed
        q[free] = p[free] / p[free].sum() * rest
    return rank, q


def zipf_bias(cfg: C.MoEConfig, key_spread: float = 0.5) -> torch.Tensor:
    """Bias whose induced load is heavy-tailed, approximately Zipf(s) over a seeded expert ranking.

    Surrogate model (not the layer's scoring): each (token, expert) key is
    z + b_e with z ~ N(0, key_spread^2) i.i.d.; then expert e is picked with
    probability Phi(b_e / key_spread) at threshold 0, and b_e is chosen so that
    this is the target q_e of zipf_target.  The realised loads are measured, not
    assumed.
    """
    _, q = zipf_target(cfg)
    b = key_spread * torch.special.ndtri(q.clamp(1e-6, 0.995))
    return b.to(torch.float32)


# ---------------------------------------------------------------- whole layer
@dataclass
class MoEInputs:
    cfg: C.MoEConfig
    x: torch.Tensor                  # [T, H] fp32 (f32 recipe) or bf16
    gate_w: torch.Tensor             # [E, H] fp32
    bias: torch.Tensor               # [E] fp32
    w13: torch.Tensor                # [E, 2I, H] fp32 / bf16 / e4m3 codes (uint8) / packed e2m1 [E, 2I, H/2]
    w2: torch.Tensor                 # [E, H, I]  likewise ([E, H, I/2] packed)
    w13_scale: torch.Tensor | None   # fp8: [E, 2I/128, H/128] fp32; MX: [E, 2I, H/32] uint8
    w2_scale: torch.Tensor | None    # fp8: [E, H/128, I/128] fp32; MX: [E, H, I/32] uint8
    shared_w13: torch.Tensor         # [S, 2Is, H] fp32 or bf16
    shared_w2: torch.Tensor          # [S, H, Is]
    norm_w: torch.Tensor | None = None   # [H] fp32 post_attention_layernorm weight (residual form)
    meta: dict = field(default_factory=dict)


def _bias(cfg):
    E = cfg.num_experts
    if cfg.bias_kind == "uniform":
        g = _gen(cfg, "bias", 0, "cpu")
        return (torch.rand(E, generator=g, dtype=torch.float32) * 2 - 1) * cfg.bias_param
    if cfg.bias_kind == "normal":
        return normal(cfg, "bias", 0, (E,), cfg.bias_param)
    if cfg.bias_kind == "zipf":
        return zipf_bias(cfg)
    raise ValueError(cfg.bias_kind)


def generate(cfg: C.MoEConfig, device="cpu", experts: bool = True) -> MoEInputs:
    """Build all inputs of one layer on `device`.  x, gate weight and bias are drawn
    on the CPU (device-independent values); expert weights are drawn on `device`."""
    T, H, E, I = cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.intermediate
    S, Is = cfg.num_shared, cfg.shared_intermediate
    act_dtype = torch.float32 if cfg.recipe == C.RECIPE_F32 else torch.bfloat16
    x = normal(cfg, "x", 0, (T, H), 1.0).to(act_dtype).to(device)
    gate_w = normal(cfg, "gate_w", 0, (E, H), cfg.gate_std).to(device)
    bias = _bias(cfg).to(device)

    w13 = w2 = w13s = w2s = None
    if experts:
        if cfg.recipe in (C.RECIPE_F32, C.RECIPE_BF16):
            w13 = torch.empty((E, 2 * I, H), dtype=act_dtype, device=device)
            w2 = torch.empty((E, H, I), dtype=act_dtype, device=device)
        elif cfg.recipe == C.RECIPE_FP8_B128:
            w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=device)
            w2 = torch.empty((E, H, I), dtype=torch.uint8, device=device)
            w13s = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
            w2s = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=device)
        elif cfg.recipe in (C.RECIPE_MXFP4, C.RECIPE_NVFP4):
            w13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
            w2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
            g = 32 if cfg.recipe == C.RECIPE_MXFP4 else 16            # scale group along K
            w13s = torch.empty((E, 2 * I, H // g), dtype=torch.uint8, device=device)
            w2s = torch.empty((E, H, I // g), dtype=torch.uint8, device=device)
        for e in range(E):
            a = normal(cfg, "w13", e, (2 * I, H), cfg.expert_std, device)
            b = normal(cfg, "w2", e, (H, I), cfg.expert_std, device)
            if cfg.recipe in (C.RECIPE_F32, C.RECIPE_BF16):
                w13[e].copy_(a.to(act_dtype))
                w2[e].copy_(b.to(act_dtype))
            elif cfg.recipe == C.RECIPE_FP8_B128:
                q, s = encode_fp8_block128(a); w13[e].copy_(q); w13s[e].copy_(s)
                q, s = encode_fp8_block128(b); w2[e].copy_(q); w2s[e].copy_(s)
            elif cfg.recipe == C.RECIPE_MXFP4:
                q, s = encode_mxfp4(a); w13[e].copy_(q); w13s[e].copy_(s)
                q, s = encode_mxfp4(b); w2[e].copy_(q); w2s[e].copy_(s)
            else:
                q, s = encode_nvfp4(a); w13[e].copy_(q); w13s[e].copy_(s)
                q, s = encode_nvfp4(b); w2[e].copy_(q); w2s[e].copy_(s)
            del a, b
    sh_dtype = torch.float32 if cfg.recipe == C.RECIPE_F32 else torch.bfloat16
    sw13 = torch.empty((S, 2 * Is, H), dtype=sh_dtype, device=device)
    sw2 = torch.empty((S, H, Is), dtype=sh_dtype, device=device)
    for s in range(S):
        sw13[s].copy_(normal(cfg, "shared_w13", s, (2 * Is, H), cfg.expert_std, device).to(sh_dtype))
        sw2[s].copy_(normal(cfg, "shared_w2", s, (H, Is), cfg.expert_std, device).to(sh_dtype))
    # RMSNorm weight of the residual form: near 1, like a trained norm
    norm_w = (1.0 + normal(cfg, "norm_w", 0, (H,), 0.1)).to(device)
    return MoEInputs(cfg, x, gate_w, bias, w13, w2, w13s, w2s, sw13, sw2, norm_w)


def expert_weight_bytes(cfg: C.MoEConfig) -> int:
    """Bytes of one routed expert's three projections plus their scales, as stored."""
    I, H = cfg.intermediate, cfg.hidden
    n = 3 * I * H
    if cfg.recipe == C.RECIPE_F32:
        return 4 * n
    if cfg.recipe == C.RECIPE_BF16:
        return 2 * n
    if cfg.recipe == C.RECIPE_FP8_B128:
        return n + 4 * (n // (128 * 128))
    if cfg.recipe == C.RECIPE_NVFP4:
        return n // 2 + n // 16
    return n // 2 + n // 32


def shared_weight_bytes(cfg: C.MoEConfig) -> int:
    n = 3 * cfg.shared_intermediate * cfg.hidden * cfg.num_shared
    return (4 if cfg.recipe == C.RECIPE_F32 else 2) * n
