"""The residual form of the layer (post_attention_layernorm in front of the MoE,
residual added in the combine) against the oracle, through the C-ABI."""
import numpy as np
import pytest
import torch

import mixture_experts_amd as M
from oracle import moe_oracle as O
from tests import harness as HN
from tests.test_gpu_parity import _check_routing
from workloads import configs as C
from workloads import generate as G

pytestmark = pytest.mark.gpu

# fp32 and bf16 rows; quantised routed activations; shared experts on the fp32
# kernel, the LDS kernel and the decode K-split slabs
RESIDUAL = [C.TINY_F32, C.MINI_F32, C.MINI_GROUPED_BF16, C.MINI_DECODE_BF16, C.MINI_PREFILL_BF16, C.MINI_FP8,
            C.MINI_MXFP4]


def _normed(inp):
    return O.rms_norm(HN.x_f64(inp), inp.norm_w.cpu().numpy(), G.RMS_EPS, inp.cfg.recipe)


def _oracle(inp, tokens=None):
    s13, s2 = HN.shared_f64(inp)
    return O.moe_forward_residual(inp.cfg, HN.x_f64(inp), inp.norm_w.cpu().numpy(), G.RMS_EPS,
                                  inp.gate_w.double().cpu().numpy(), inp.bias.cpu().numpy(), HN.expert_raw_fn(inp),
                                  s13, s2, tokens=tokens)


def _run(inp, resid=None, out=None):
    cfg = M.make_config(inp.cfg)
    b = M.alloc_buffers(cfg, inp.x.device)
    ex, sh = HN.weights(inp)
    resid = inp.x if resid is None else resid
    out = b.out if out is None else out
    M.moe_forward_residual(cfg, resid, inp.norm_w, G.RMS_EPS, inp.gate_w, inp.bias, ex, sh, out, b.topk_idx,
                           b.topk_w, b.ws)
    torch.cuda.synchronize()
    return b, out


@pytest.mark.parametrize("cfg", RESIDUAL, ids=lambda c: c.name)
def test_rmsnorm_rows_are_bit_exact(cfg):
    inp = G.generate(cfg, device="cuda")
    x = torch.empty_like(inp.x)
    M.moe_rmsnorm(M.make_config(cfg), inp.x, inp.norm_w, G.RMS_EPS, x)
    torch.cuda.synchronize()
    want = O.rms_norm(HN.x_f64(inp), inp.norm_w.cpu().numpy(), G.RMS_EPS, cfg.recipe)
    got = HN.out_f64(x)
    assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} values differ"


@pytest.mark.parametrize("cfg", RESIDUAL, ids=lambda c: c.name)
def test_forward_residual_parity(cfg):
    inp = G.generate(cfg, device="cuda")
    b, out = _run(inp)
    ref = _oracle(inp)
    _check_routing(b, ref, inp, _normed(inp))
    err = HN.rel_l2(HN.out_f64(out), ref["out"])
    assert err < HN.TOL[cfg.recipe], f"out rel-L2 {err:.3e}"
    # the residual is really there: the result differs from the MoE output alone
    assert HN.rel_l2(ref["out"], ref["moe_out"]) > 0.1
    # in place: out written over the residual buffer itself
    h = inp.x.clone()
    _run(inp, resid=h, out=h)
    assert torch.equal(h, out)


def test_forward_residual_full_size_decode():
    cfg = C.DECODE_BF16
    torch.cuda.empty_cache()
    inp = G.generate(cfg, device="cuda")
    b, out = _run(inp)
    tokens = HN.sample_tokens(cfg.num_tokens, 24)
    ref = _oracle(inp, tokens=tokens)
    _check_routing(b, ref, inp, _normed(inp))
    got = HN.out_f64(out[torch.from_numpy(tokens).cuda()])
    err = HN.rel_l2(got, ref["out"])
    rows = HN.row_rel_l2(got, ref["out"])
    print(f"{cfg.name} residual form: {tokens.size} tokens, out rel-L2 {err:.3e}, worst row {rows.max():.3e}")
    assert err < HN.TOL[cfg.recipe], err
    assert rows.max() < 5 * HN.TOL[cfg.recipe], rows.max()
    del inp, b
    torch.cuda.empty_cache()
