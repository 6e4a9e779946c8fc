"""moe_forward against the oracle on seeded random layer shapes: every recipe,
ragged token, hidden, intermediate and expert counts, grouped and ungrouped
selection, 0-2 shared experts, both score functions, the method flags, and token
counts on both sides of the screened gate's threshold (512).  Routing indices
bit-exact, weights within the recipe's bound (check_routing), and the outputs of
all tokens within the recipe's relative-L2 tolerance, the worst single row
within 5x it.  The CPU test checks that every drawn shape is one the library
accepts, so the GPU test runs only shapes the kernels are built for."""
import numpy as np
import pytest
import torch

import mixture_experts_amd as M
from tests import harness as HN
from workloads import configs as C
from workloads import generate as G

N_PER_RECIPE = 6
RECIPES = [C.RECIPE_F32, C.RECIPE_BF16, C.RECIPE_FP8_B128, C.RECIPE_MXFP4, C.RECIPE_NVFP4]


def _draw(recipe: int, i: int) -> C.MoEConfig:
    rng = np.random.default_rng(1000 * recipe + i)
    q = 32 if recipe == C.RECIPE_F32 else (256 if recipe in (C.RECIPE_MXFP4, C.RECIPE_NVFP4) else 128)
    qs = 32 if recipe == C.RECIPE_F32 else 128
    H = q * int(rng.integers(1, 768 // q + 1))
    I = q * int(rng.integers(1, 512 // q + 1))
    E = int(rng.choice([1, 2, 5, 8, 12, 24, 33, 48, 64, 96]))
    k = int(rng.integers(1, min(16, E) + 1))
    n_group, topk_group = 1, 1
    divs = [d for d in (2, 3, 4, 8) if E % d == 0 and E // d >= 2]
    if divs and rng.random() < 0.5:
        n_group = int(rng.choice(divs))
        per = E // n_group
        lo = -(-k // per)                                   # enough kept groups to hold k experts
        topk_group = int(rng.integers(lo, n_group + 1))
    if recipe == C.RECIPE_F32:
        T = int(rng.integers(1, 200))
    else:
        T = int(rng.choice([1, 7, 64, 130, 300, 511, 512, 600, 700]))
    ns = int(rng.integers(0, 3))
    bias_kind = str(rng.choice(["normal", "uniform", "zipf"]))
    SI = qs * int(rng.integers(1, 384 // qs + 1)) if ns else 0
    return C.MoEConfig(
        name=f"rand_{C.RECIPE_NAMES[recipe]}_{i}", num_tokens=T, hidden=H, num_experts=E, top_k=k,
        intermediate=I, num_shared=ns, shared_intermediate=SI, n_group=n_group, topk_group=topk_group,
        score_func=int(rng.integers(0, 2)), norm_topk_prob=bool(rng.random() < 0.75),
        routed_scaling_factor=float(rng.choice([1.0, 2.5, 2.827])), recipe=recipe,
        swiglu_limit=float(rng.choice([0.0, 0.0, 7.0, 0.5])), seed=int(rng.integers(0, 1 << 30)),
        gate_std=1.0 / 16.0, bias_kind=bias_kind,
        bias_param=1.1 if bias_kind == "zipf" else float(rng.choice([0.01, 0.1])))


CASES = [_draw(r, i) for r in RECIPES for i in range(N_PER_RECIPE)]


def test_drawn_shapes_are_accepted_by_the_library():
    for cfg in CASES:
        assert M.moe_workspace_bytes(M.make_config(cfg)) > 0, cfg


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_random_shape_matches_the_oracle(cfg):
    print(f"case {cfg}", flush=True)
    inp = G.generate(cfg, device="cuda")
    b = HN.run_forward(inp)
    ref = HN.oracle(inp)
    HN.check_routing(cfg, b.topk_idx.cpu().numpy(), b.topk_w.cpu().numpy(), ref["routing"], HN.x_f64(inp),
                     inp.gate_w.cpu().numpy())
    got, want = HN.out_f64(b.out), ref["out"]
    tol = HN.TOL[cfg.recipe]
    err = HN.rel_l2(got, want)
    rows = HN.row_rel_l2(got, want)
    print(f"{cfg.name}: rel-L2 {err:.3e}, worst row {rows.max():.3e}", flush=True)
    assert err < tol, err
    assert rows.max() < 5 * tol, (rows.max(), int(rows.argmax()))
    del inp, b
    torch.cuda.empty_cache()
