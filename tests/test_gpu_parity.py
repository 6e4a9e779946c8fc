"""HIP path vs the CPU oracle, through the C-ABI, on seeded inputs.

Small workloads: every stage, element by element (indices and permutation
bit-exact, quantised activation bytes bit-exact, outputs within the recipe's
relative-L2 tolerance).  Full-size workloads, in the launch configuration the
benchmark times (moe_forward): all routing indices bit-exact, the permutation
bit-exact, and the outputs of sampled tokens within tolerance."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests import harness as HN
from workloads import configs as C
from workloads import generate as G

pytestmark = pytest.mark.gpu

SMALL = [C.TINY_F32] + C.MINI_CONFIGS


def _check_routing(b, ref, inp, x64=None):
    """x64: the gate's input rows, when they are not inp.x (the residual form's norm)."""
    HN.check_routing(inp.cfg, b.topk_idx.cpu().numpy(), b.topk_w.cpu().numpy(), ref["routing"],
                     HN.x_f64(inp) if x64 is None else x64, inp.gate_w.cpu().numpy())


def _check_permutation(b, ref):
    p = ref["perm"]
    assert np.array_equal(b.offsets.cpu().numpy(), p["offsets"])
    assert np.array_equal(b.sorted_pair.cpu().numpy(), p["sorted_pair"])
    assert np.array_equal(b.pair_pos.cpu().numpy(), p["pair_pos"])


def _check_x_perm(inp, b, ref):
    cfg = inp.cfg
    x32 = HN.x_f64(inp).astype(np.float32)
    rows, scales = O.gather_rows(cfg.recipe, x32, ref["perm"]["sorted_pair"], cfg.top_k)
    got = HN.to_np(b.x_perm)
    if cfg.recipe == C.RECIPE_F32:
        assert np.array_equal(got, rows)
    elif cfg.recipe == C.RECIPE_BF16:
        assert np.array_equal(O.decode_bf16(got), rows.astype(np.float64))
    elif cfg.recipe == C.RECIPE_NVFP4:
        assert np.array_equal(got.astype(np.float64), rows), f"{(got.astype(np.float64) != rows).sum()} values differ"
    else:
        assert np.array_equal(got, rows), f"{(got != rows).sum()} code bytes differ"
        assert np.array_equal(HN.to_np(b.x_perm_scale), scales)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_stagewise_parity_small(cfg):
    inp = G.generate(cfg, device="cuda")
    b = HN.run_stages(inp)
    ref = HN.oracle(inp)
    _check_routing(b, ref, inp)
    _check_permutation(b, ref)
    _check_x_perm(inp, b, ref)
    tol = HN.TOL[cfg.recipe]
    # y_perm rows against the oracle's per-(token, slot) expert outputs
    y = HN.out_f64(b.y_perm)
    pos = ref["perm"]["pair_pos"].reshape(cfg.num_tokens, cfg.top_k)
    err_y = HN.rel_l2(y[pos], ref["y"])
    assert err_y < tol, f"y_perm rel-L2 {err_y:.3e}"
    err = HN.rel_l2(HN.out_f64(b.out), ref["out"])
    assert err < tol, f"out rel-L2 {err:.3e}"
    # the fused entry point runs the same kernels: identical bits
    b2 = HN.run_forward(inp)
    assert torch.equal(b2.out, b.out)
    assert torch.equal(b2.topk_idx, b.topk_idx)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_runs_are_bit_identical(cfg):
    inp = G.generate(cfg, device="cuda")
    a = HN.run_forward(inp)
    out1 = a.out.clone()
    HN.run_forward(inp, a)
    assert torch.equal(out1, a.out)


# Method variants (norm_topk_prob = false; swiglu_limit > 0) on workloads that
# between them take every SwiGLU epilogue: register-streaming bf16/fp8/MX tiles,
# LDS-staged bf16/fp8 tiles, the fp32 kernel and the decode shared expert's
# K-split slabs.  The limit clips a large share of the gate and up values
# (their standard deviation is about 0.4 at these sizes).
VARIANTS = [
    (C.MINI_GROUPED_BF16, dict(swiglu_limit=0.25)),
    (C.MINI_DECODE_BF16, dict(swiglu_limit=0.25)),
    (C.MINI_MIXED_BF16, dict(swiglu_limit=0.25)),
    (C.MINI_FP8, dict(swiglu_limit=0.25)),
    (C.MINI_MXFP4, dict(swiglu_limit=0.25)),
    (C.MINI_MXFP4_WIDE, dict(swiglu_limit=0.25)),
    (C.MINI_NVFP4, dict(swiglu_limit=0.25)),
    (C.MINI_F32, dict(swiglu_limit=0.2)),
    (C.MINI_GROUPED_BF16, dict(norm_topk_prob=False)),
    (C.MINI_FP8, dict(norm_topk_prob=False)),
    (C.TINY_F32, dict(norm_topk_prob=False, swiglu_limit=0.2)),
]


def _parity_both_paths(inp):
    """Stage-wise and fused paths against the oracle; returns the oracle's result."""
    b = HN.run_stages(inp)
    ref = HN.oracle(inp)
    _check_routing(b, ref, inp)
    _check_permutation(b, ref)
    tol = HN.TOL[inp.cfg.recipe]
    err = HN.rel_l2(HN.out_f64(b.out), ref["out"])
    assert err < tol, f"out rel-L2 {err:.3e}"
    b2 = HN.run_forward(inp)
    assert torch.equal(b2.out, b.out)
    return ref


@pytest.mark.parametrize("case", VARIANTS,
                         ids=lambda c: c[0].name + "-" + ",".join(f"{k}={v}" for k, v in c[1].items()))
def test_method_variants(case):
    base, kw = case
    cfg = base.replace(**kw)
    inp = G.generate(cfg, device="cuda")             # same tensors as the base workload (same name)
    ref = _parity_both_paths(inp)
    # the variant changes the result well beyond the tolerance
    ref0 = HN.oracle(dataclasses.replace(inp, cfg=base))
    assert HN.rel_l2(ref["out"], ref0["out"]) > 5 * HN.TOL[cfg.recipe]


SHAPES = [
    # smallest fp4 shapes: one 256-deep stage per gate/up tile (and one NVFP4 / two
    # 128-deep MXFP4 down stages), so every register ring runs past its last stage
    C.MINI_MXFP4.replace(name="mini_mxfp4_h256", hidden=256, intermediate=256),
    C.MINI_NVFP4.replace(name="mini_nvfp4_h256", hidden=256, intermediate=256),
    # token counts whose average rows per expert select the register-streaming
    # tile heights no other workload reaches: bf16 64 rows (40 < avg <= 48), fp8
    # 32 and 64 rows, MXFP4 32 rows (avg <= 24)
    C.MINI_GROUPED_BF16.replace(name="mini_grouped_bf16_t240", num_tokens=240),
    C.MINI_FP8.replace(name="mini_fp8_t40", num_tokens=40),
    C.MINI_FP8.replace(name="mini_fp8_t180", num_tokens=180),
    C.MINI_MXFP4.replace(name="mini_mxfp4_t64", num_tokens=64),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_more_shapes(cfg):
    _parity_both_paths(G.generate(cfg, device="cuda"))


# The LDS-staged kernels (and the register-streaming kernel for MXFP4 / NVFP4)
# copy through buffer descriptors (32-bit offsets) when A and the expert weights
# fit 4 GiB, else with 64-bit FLAT copies.  No test shape reaches the second form,
# so these cases run the library build that forces it (libmoe_mi355x_flatcopy.so).
@pytest.mark.parametrize("cfg", [C.MINI_PREFILL_BF16, C.MINI_PREFILL_FP8, C.MINI_MIXED_BF16, C.MINI_MXFP4_WIDE,
                                 C.MINI_NVFP4, C.MINI_SKEWED_FP8], ids=lambda c: c.name)
def test_lds_flat_copy_form(cfg):
    import mixture_experts_amd as M
    with M.library(M.FLAT_LIB_PATH):
        _parity_both_paths(G.generate(cfg, device="cuda"))


def _edge_inputs(kind):
    cfg = C.MINI_GROUPED_BF16
    if kind == "single_token":
        cfg = cfg.replace(num_tokens=1)
    inp = G.generate(cfg, device="cuda")
    if kind == "one_hot_expert":           # every token picks expert 5 (and 3 more)
        inp.bias[5] += 10.0
    if kind == "exact_ties":               # twins 3/9 and 20/21: identical gate rows and bias
        inp.gate_w[9] = inp.gate_w[3]; inp.bias[9] = inp.bias[3]
        inp.gate_w[21] = inp.gate_w[20]; inp.bias[21] = inp.bias[20]
    if kind == "all_tied":                 # one gate row for every expert, zero bias
        inp.gate_w[:] = inp.gate_w[0]; inp.bias.zero_()
    return inp


@pytest.mark.parametrize("kind", ["single_token", "one_hot_expert", "exact_ties", "all_tied"])
def test_edge_cases(kind):
    inp = _edge_inputs(kind)
    b = HN.run_stages(inp)
    ref = HN.oracle(inp)
    _check_routing(b, ref, inp)
    _check_permutation(b, ref)
    err = HN.rel_l2(HN.out_f64(b.out), ref["out"])
    assert err < HN.TOL[inp.cfg.recipe], err
    if kind == "all_tied":
        k, n = inp.cfg.top_k, inp.cfg.n_group
        assert np.all(b.topk_idx.cpu().numpy() == np.arange(k))


@pytest.mark.parametrize("cfg", C.FULL_CONFIGS[1:] + C.NEXT_CONFIGS, ids=lambda c: c.name)
def test_full_size_parity(cfg):
    """Full size, in the benchmark's launch configuration.  Every token's routing and
    the whole permutation are bit-exact.  Outputs are compared on every token when
    T <= 256, else on tokens that together reach every expert and the first and last
    row of every 256-row tile of the three largest experts: pooled rel-L2 within the
    tolerance and the worst single row within 5x it."""
    torch.cuda.empty_cache()
    inp = G.generate(cfg, device="cuda")
    b = HN.run_forward(inp)
    ref_r = O.route(cfg, HN.x_f64(inp), inp.gate_w.double().cpu().numpy(), inp.bias.cpu().numpy())
    perm = O.permute(ref_r["idx"], cfg.num_experts)
    _check_routing(b, {"routing": ref_r}, inp)
    # permutation of the full routing through the stand-alone entry point
    import mixture_experts_amd as M
    M.moe_permute(b.cfg, b.topk_idx, inp.x, b.offsets, b.sorted_pair, b.pair_pos, b.x_perm, b.x_perm_scale, b.ws)
    torch.cuda.synchronize()
    _check_permutation(b, {"perm": perm})
    if cfg.num_tokens <= 256:
        tokens = np.arange(cfg.num_tokens)
    else:
        tokens = HN.cover_tokens(ref_r["idx"], perm["offsets"], perm["sorted_pair"])
    touched = np.unique(ref_r["idx"][tokens])
    assert touched.size == np.count_nonzero(np.diff(perm["offsets"]))   # every expert with rows is checked
    want = HN.oracle_tokens(inp, tokens, ref_r, perm)
    got = HN.out_f64(b.out[torch.from_numpy(tokens).cuda()])
    err = HN.rel_l2(got, want)
    rows = HN.row_rel_l2(got, want)
    print(f"{cfg.name}: {tokens.size} tokens over {touched.size} experts, out rel-L2 {err:.3e}, "
          f"worst row {rows.max():.3e} (token {tokens[rows.argmax()]})")
    tol = HN.TOL[cfg.recipe]
    assert err < tol, err
    assert rows.max() < 5 * tol, (rows.max(), tokens[rows.argmax()])
    del inp, b
    torch.cuda.empty_cache()
