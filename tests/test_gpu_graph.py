"""The layer call under HIP graph capture: moe_forward and moe_forward_noalloc
enqueue only kernel launches on the caller's stream (no allocation, no memset, no
host synchronisation), so a serving loop can capture one call and replay it.
Each case captures one call through the C-ABI (torch.cuda.graph drives the
capture), then replays it several times with new token rows copied into the
captured input buffer and eager layer calls on the same workspace in between;
every replay must give the eager call's bits on the same rows (the kernels are
deterministic)."""
import pytest
import torch

import mixture_experts_amd as M
from tests import harness as HN
from workloads import configs as C
from workloads import generate as G

pytestmark = pytest.mark.gpu

CASES = [C.MINI_DECODE_BF16, C.MINI_PREFILL_BF16, C.MINI_FP8, C.MINI_MXFP4, C.DECODE_BF16]
REPLAYS = 3


def _rows(x, i):
    """Token rows for replay i: a seeded permutation of the rows, scaled."""
    g = torch.Generator(device="cpu").manual_seed(100 + i)
    perm = torch.randperm(x.shape[0], generator=g).to(x.device)
    return (x[perm].float() * (1.0 + 0.25 * i)).to(x.dtype)


@pytest.mark.parametrize("noalloc", [False, True], ids=["moe_forward", "moe_forward_noalloc"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_captured_call_replays_the_eager_result(cfg, noalloc):
    print(f"graph {cfg.name} noalloc={noalloc}", flush=True)
    inp = G.generate(cfg, device="cuda")
    mcfg = M.make_config(cfg)
    if noalloc and M.moe_workspace_bytes(mcfg) > M.moe_forward_noalloc_scratch_bytes():
        pytest.skip("beyond the no-alloc scratch")
    ex, sh = HN.weights(inp)
    b = M.alloc_buffers(mcfg, "cuda")
    x = inp.x.clone()                                   # the captured input buffer
    out = torch.empty_like(b.out)
    idx = torch.empty_like(b.topk_idx)
    w = torch.empty_like(b.topk_w)

    def call(xx, o, i, ww):
        if noalloc:
            M.moe_forward_noalloc(mcfg, xx, inp.gate_w, inp.bias, ex, sh, o, i, ww)
        else:
            M.moe_forward(mcfg, xx, inp.gate_w, inp.bias, ex, sh, o, i, ww, b.ws)

    call(x, out, idx, w)                                # eager first: first-launch work stays out of the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x, out, idx, w)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        rows = _rows(inp.x, i)
        ref_out, ref_idx, ref_w = torch.empty_like(out), torch.empty_like(idx), torch.empty_like(w)
        call(rows, ref_out, ref_idx, ref_w)             # eager, same workspace
        torch.cuda.synchronize()
        x.copy_(rows)
        out.fill_(float("nan"))
        idx.fill_(-1)
        w.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), i
        assert torch.equal(w, ref_w), i
        assert torch.equal(out, ref_out), i
    del graph
    torch.cuda.synchronize()
