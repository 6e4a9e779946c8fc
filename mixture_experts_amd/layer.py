"""Device buffers for one MoE layer call (torch allocations: memory plumbing only)."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class MoELayerBuffers:
    cfg: _lib.MoeConfig
    topk_idx: torch.Tensor      # [T, k] int32
    topk_w: torch.Tensor        # [T, k] fp32
    offsets: torch.Tensor       # [E+1] int32
    sorted_pair: torch.Tensor   # [T*k] int32
    pair_pos: torch.Tensor      # [T*k] int32
    x_perm: torch.Tensor        # [T*k, H] fp32 / bf16 / uint8 codes
    x_perm_scale: torch.Tensor | None
    y_perm: torch.Tensor        # [T*k, H] fp32 / bf16
    out: torch.Tensor           # [T, H] fp32 / bf16
    ws: torch.Tensor            # uint8 workspace


def alloc_buffers(cfg: _lib.MoeConfig, device="cuda") -> MoELayerBuffers:
    T, H, E, k = cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k
    P = T * k
    f32 = cfg.recipe == _lib.RECIPE_F32
    act = torch.float32 if f32 else torch.bfloat16
    if cfg.recipe in (_lib.RECIPE_F32, _lib.RECIPE_BF16):
        x_perm = torch.empty((P, H), dtype=act, device=device)
        x_perm_scale = None
    elif cfg.recipe == _lib.RECIPE_NVFP4:                  # fp16 values of the NVFP4 rows
        x_perm = torch.empty((P, H), dtype=torch.float16, device=device)
        x_perm_scale = None
    elif cfg.recipe == _lib.RECIPE_FP8_B128:
        x_perm = torch.empty((P, H), dtype=torch.uint8, device=device)
        x_perm_scale = torch.empty((P, H // 128), dtype=torch.float32, device=device)
    else:
        x_perm = torch.empty((P, H), dtype=torch.uint8, device=device)
        x_perm_scale = torch.empty((P, H // 32), dtype=torch.uint8, device=device)
    nbytes = _lib.moe_workspace_bytes(cfg)
    if nbytes == 0:
        raise _lib.MoeError("configuration rejected by moe_workspace_bytes")
    return MoELayerBuffers(
        cfg=cfg,
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=device),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
        offsets=torch.empty((E + 1,), dtype=torch.int32, device=device),
        sorted_pair=torch.empty((P,), dtype=torch.int32, device=device),
        pair_pos=torch.empty((P,), dtype=torch.int32, device=device),
        x_perm=x_perm, x_perm_scale=x_perm_scale,
        y_perm=torch.empty((P, H), dtype=act, device=device),
        out=torch.empty((T, H), dtype=act, device=device),
        ws=torch.empty((nbytes,), dtype=torch.uint8, device=device),
    )
