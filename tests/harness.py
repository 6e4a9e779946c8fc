"""Shared helpers for the parity tests: run the HIP path through the C-ABI and the
oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_amd as M
from oracle import moe_oracle as O
from workloads import configs as C
from workloads import generate as G

# NVFP4: the same bound as the other quantised recipes (the oracle emulates the
# quantisation; what remains is fp32 summation order, bf16 outputs and the rare
# activation code decided differently by those last bits)
TOL = {C.RECIPE_F32: 1e-5, C.RECIPE_BF16: 2e-2, C.RECIPE_FP8_B128: 6e-2, C.RECIPE_MXFP4: 6e-2, C.RECIPE_NVFP4: 6e-2}


def to_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in its storage form (bf16 as uint16 bit patterns)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def x_f64(inp: G.MoEInputs) -> np.ndarray:
    x = to_np(inp.x)
    return O.decode_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64)


def expert_raw_fn(inp: G.MoEInputs):
    def raw(e: int) -> dict:
        d = {"w13": to_np(inp.w13[e]), "w2": to_np(inp.w2[e])}
        if inp.w13_scale is not None:
            d["w13_scale"] = to_np(inp.w13_scale[e])
            d["w2_scale"] = to_np(inp.w2_scale[e])
        return d
    return raw


def shared_f64(inp: G.MoEInputs):
    a, b = to_np(inp.shared_w13), to_np(inp.shared_w2)
    if a.dtype == np.uint16:
        return O.decode_bf16(a), O.decode_bf16(b)
    return a.astype(np.float64), b.astype(np.float64)


def out_f64(t: torch.Tensor) -> np.ndarray:
    a = to_np(t)
    return O.decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def weights(inp: G.MoEInputs):
    ex = M.make_expert_weights(inp.cfg.recipe, inp.w13, inp.w2, inp.w13_scale, inp.w2_scale)
    sh = M.make_weights(inp.shared_w13, inp.shared_w2) if inp.cfg.num_shared > 0 else None
    return ex, sh


def run_stages(inp: G.MoEInputs, bufs=None):
    """route -> permute -> grouped_ffn -> combine through the C-ABI; returns the buffers."""
    cfg = M.make_config(inp.cfg)
    b = bufs or M.alloc_buffers(cfg, inp.x.device)
    ex, sh = weights(inp)
    M.moe_route(cfg, inp.x, inp.gate_w, inp.bias, b.topk_idx, b.topk_w, b.ws)
    M.moe_permute(cfg, b.topk_idx, inp.x, b.offsets, b.sorted_pair, b.pair_pos, b.x_perm, b.x_perm_scale, b.ws)
    M.moe_grouped_ffn(cfg, b.offsets, b.x_perm, b.x_perm_scale, ex, b.y_perm, b.ws)
    M.moe_combine(cfg, b.y_perm, b.pair_pos, b.topk_w, inp.x, sh, b.out, b.ws)
    torch.cuda.synchronize()
    return b


def run_forward(inp: G.MoEInputs, bufs=None):
    cfg = M.make_config(inp.cfg)
    b = bufs or M.alloc_buffers(cfg, inp.x.device)
    ex, sh = weights(inp)
    M.moe_forward(cfg, inp.x, inp.gate_w, inp.bias, ex, sh, b.out, b.topk_idx, b.topk_w, b.ws)
    torch.cuda.synchronize()
    return b


def oracle(inp: G.MoEInputs, tokens=None):
    cfg = inp.cfg
    s13, s2 = shared_f64(inp)
    return O.moe_forward(cfg, x_f64(inp), inp.gate_w.double().cpu().numpy(), inp.bias.cpu().numpy(),
                         expert_raw_fn(inp), s13, s2, tokens=tokens)


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and random tokens (sorted, unique)."""
    rng = np.random.default_rng(seed)
    pick = set([0, T - 1]) | set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(pick)[:max(n, 2)])
