"""Routing with bf16 activations at 512 tokens or more, where the gate runs as a
bf16-MFMA screen plus an exact recompute of the logits that can change the
selection, against the oracle through moe_route: every index bit-exact, and the
weights within the screen's error bound (those of recomputed picks are exact).
The shapes reach the screen's edges: ragged token and expert tiles, an expert
count that is not a multiple of 4, grouped selection, the largest expert count, a
K split across many blocks, rows of 512 to 8192 (one to four 2048-wide passes of
the exact recompute), and ties that only an exact recompute can order."""
import numpy as np
import pytest
import torch

import mixture_experts_amd as M
from oracle import moe_oracle as O
from tests import harness as HN
from workloads import configs as C
from workloads import generate as G

pytestmark = pytest.mark.gpu


def _cfg(name, T, H, E, k, **kw):
    base = dict(intermediate=256, num_shared=0, shared_intermediate=0, recipe=C.RECIPE_BF16, gate_std=0.02)
    base.update(kw)
    return C.MoEConfig(name=name, num_tokens=T, hidden=H, num_experts=E, top_k=k, **base)


CASES = [
    _cfg("screen_grouped", 777, 1024, 256, 8, n_group=8, topk_group=4, routed_scaling_factor=2.5),
    _cfg("screen_sqrtsoftplus_e200", 600, 2048, 200, 6, score_func=C.SCORE_SQRTSOFTPLUS,
         routed_scaling_factor=2.5, recipe=C.RECIPE_FP8_B128, bias_kind="zipf", bias_param=1.1),
    _cfg("screen_h7168", 640, 7168, 384, 8, recipe=C.RECIPE_MXFP4),
    _cfg("screen_ksplit", 512, 7168, 128, 8),                  # 4 tiles: the K range split over many blocks
    _cfg("screen_e1024", 512, 512, 1024, 16, n_group=16, topk_group=8),
    _cfg("screen_h6144", 520, 6144, 64, 4, norm_topk_prob=False),
    _cfg("screen_h4096", 530, 4096, 32, 4, recipe=C.RECIPE_NVFP4),
    _cfg("screen_h8192", 515, 8192, 40, 5, score_func=C.SCORE_SQRTSOFTPLUS),
]


def _route(inp):
    cfg = M.make_config(inp.cfg)
    T, k = inp.cfg.num_tokens, inp.cfg.top_k
    ws = torch.empty(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route(cfg, inp.x, inp.gate_w, inp.bias, idx, w, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


def _check(inp):
    idx, w = _route(inp)
    x64 = inp.x.float().cpu().double().numpy()
    gate_w = inp.gate_w.cpu().numpy()
    ref = O.route(inp.cfg, x64, gate_w.astype(np.float64), inp.bias.cpu().numpy())
    HN.check_routing(inp.cfg, idx, w, ref, x64, gate_w)
    return idx


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_screened_routing(cfg):
    print(f"case {cfg.name}", flush=True)
    _check(G.generate(cfg, device="cuda", experts=False))


@pytest.mark.parametrize("kind", ["exact_ties", "all_tied", "one_hot_expert", "zero_rows", "large_x"])
def test_screened_routing_edges(kind):
    cfg = CASES[0]
    print(f"case {kind}", flush=True)
    inp = G.generate(cfg, device="cuda", experts=False)
    if kind == "exact_ties":               # twins with identical gate rows and bias, one pair per group
        for a, b in [(3, 9), (20, 21), (100, 101), (200, 255)]:
            inp.gate_w[b] = inp.gate_w[a]
            inp.bias[b] = inp.bias[a]
    if kind == "all_tied":                 # one gate row for every expert, zero bias
        inp.gate_w[:] = inp.gate_w[0]
        inp.bias.zero_()
    if kind == "one_hot_expert":
        inp.bias[77] += 10.0
    if kind == "zero_rows":                # all logits exactly 0: the bias alone decides
        inp.x[::7] = 0
    if kind == "large_x":
        inp.x.mul_(1000.0)
    idx = _check(inp)
    if kind == "all_tied":
        assert np.all(idx == np.arange(cfg.top_k))
    if kind == "one_hot_expert":
        assert np.all((idx == 77).any(axis=1))
