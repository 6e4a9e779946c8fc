"""moe_forward_noalloc (the entry point with a static scratch array) against
moe_forward through the C-ABI: identical outputs and routing on two calls in a row,
the second with a smaller input; configurations beyond the array are rejected."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_amd as M
from mixture_experts_amd import _lib as L
from tests import harness as HN
from workloads import configs as C
from workloads import generate as G

pytestmark = pytest.mark.gpu


def _both(cfg):
    inp = G.generate(cfg, device="cuda")
    ref = HN.run_forward(inp)                          # moe_forward with a workspace
    mcfg = M.make_config(cfg)
    ex, sh = HN.weights(inp)
    out = torch.full_like(ref.out, float("nan"))
    idx = torch.full_like(ref.topk_idx, -1)
    w = torch.full_like(ref.topk_w, float("nan"))
    M.moe_forward_noalloc(mcfg, inp.x, inp.gate_w, inp.bias, ex, sh, out, idx, w)
    torch.cuda.synchronize()
    return inp, ref, out, idx, w


@pytest.mark.parametrize("first,second", [(C.DECODE_BF16, C.MINI_DECODE_BF16), (C.MINI_MXFP4, C.TINY_F32),
                                          (C.MINI_FP8, C.MINI_GROUPED_BF16)], ids=lambda c: c.name)
def test_noalloc_matches_moe_forward_twice(first, second):
    for cfg in (first, second):
        print(f"noalloc {cfg.name}", flush=True)
        assert M.moe_workspace_bytes(M.make_config(cfg)) <= M.moe_forward_noalloc_scratch_bytes()
        inp, ref, out, idx, w = _both(cfg)
        assert torch.equal(idx, ref.topk_idx)
        assert torch.equal(w, ref.topk_w)
        assert torch.equal(out, ref.out)                 # same kernels, same inputs: the same bits
        # and within the recipe's tolerance of the oracle on a few tokens
        tokens = HN.sample_tokens(cfg.num_tokens, 4)
        want = HN.oracle(inp, tokens=tokens)["out"]
        assert HN.rel_l2(HN.out_f64(out[torch.from_numpy(tokens).cuda()]), want) < HN.TOL[cfg.recipe]
        del inp, ref
        torch.cuda.empty_cache()


def test_noalloc_rejects_configurations_beyond_its_scratch():
    cfg = M.make_config(C.PREFILL_BF16_GROUPED)
    assert M.moe_workspace_bytes(cfg) > M.moe_forward_noalloc_scratch_bytes()
    lib = M.load()
    st = lib.moe_forward_noalloc(ctypes.byref(cfg), None, None, None, None, None, None, None, None, None)
    assert st == L.MOE_ERR_WORKSPACE_TOO_SMALL
    bad = M.make_config(C.TINY_F32.replace(top_k=0))
    assert lib.moe_forward_noalloc(ctypes.byref(bad), None, None, None, None, None, None, None, None, None) == L.MOE_ERR_INVALID_ARGUMENT
