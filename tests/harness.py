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


# The library screens the gate logits on the bf16 MFMA pipe when the activations are
# bf16 and there are at least this many tokens; picks whose rank the screen leaves
# in no doubt then take their weight from the screened logit.
SCREEN_MIN_TOKENS = 512


def gate_screened(cfg) -> bool:
    return cfg.recipe != C.RECIPE_F32 and cfg.num_tokens >= SCREEN_MIN_TOKENS


def _bf16_rn(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _ulp32(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float32))
    return np.spacing(np.maximum(a, np.float32(2.0 ** -126))).astype(np.float64)


def screened_weight_bound(cfg, x64: np.ndarray, gate_w: np.ndarray, ref: dict) -> np.ndarray:
    """Per pick, the largest |w - w_exact| for a weight computed from a screened logit.

    The screen splits each fp32 gate weight (round to nearest) into two bf16 pieces
    and a remainder, w = w1 + w2 + w3, and adds the exact products with the pieces in
    fp32 (256 per accumulator group, then the groups); its logit is within
    eps = gamma_n |x|_2 (|w1|_2 + |w2|_2) + |x|_2 |w3|_2 of the exact one, with
    n = 256 + H/128 + 2 (the most groups any K split has).  The score is then within
    lip (eps + ulp(l)) + ulp(s), lip = 1/4 (sigmoid) or 0.32 (sqrt(softplus)), and the
    normalised, scaled weights move by at most the first-order sum below plus two
    roundings."""
    w32 = np.asarray(gate_w, dtype=np.float32)
    w1 = _bf16_rn(w32)
    r = (w32 - w1).astype(np.float32)
    w2 = _bf16_rn(r)
    w3 = (r - w2).astype(np.float32)
    n12 = np.linalg.norm(w1.astype(np.float64), axis=1) + np.linalg.norm(w2.astype(np.float64), axis=1)
    n3 = np.linalg.norm(w3.astype(np.float64), axis=1)
    xn = np.linalg.norm(x64, axis=1)
    u, n = 2.0 ** -24, 256 + cfg.hidden // 128 + 2
    gam = n * u / (1 - n * u)
    lip = 0.25 if cfg.score_func == C.SCORE_SIGMOID else 0.32
    idx = ref["idx"]
    eps = gam * xn[:, None] * n12[idx] + xn[:, None] * n3[idx]
    logit = np.take_along_axis(ref["logits"], idx, axis=1)
    s = np.take_along_axis(ref["s"], idx, axis=1).astype(np.float64)
    ds = lip * (eps + _ulp32(logit)) + _ulp32(s)
    scale = float(cfg.routed_scaling_factor)
    if cfg.norm_topk_prob:
        S = s.sum(axis=1, keepdims=True)
        dw = scale * (ds / S + s * ds.sum(axis=1, keepdims=True) / S ** 2)
    else:
        dw = scale * ds
    return dw * 1.001 + 2 * _ulp32(ref["w"])


def check_routing(cfg, idx: np.ndarray, w: np.ndarray, ref: dict, x64=None, gate_w=None):
    """Indices bit-exact; weights to 1e-6 relative, or, for a screened gate, within
    screened_weight_bound with a median relative error below 1e-6."""
    bad = np.nonzero((idx != ref["idx"]).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens routed differently, first {bad[:5]}: {idx[bad[:2]]} vs {ref['idx'][bad[:2]]}"
    if not gate_screened(cfg):
        np.testing.assert_allclose(w, ref["w"], rtol=1e-6, atol=0)
        return
    bound = screened_weight_bound(cfg, x64, gate_w, ref)
    dev = np.abs(w.astype(np.float64) - ref["w"].astype(np.float64))
    worst = np.unravel_index(np.argmax(dev / bound), dev.shape)
    assert np.all(dev <= bound), f"weight {worst}: |dw| {dev[worst]:.3e} > bound {bound[worst]:.3e}"
    rel = dev / np.abs(ref["w"]).astype(np.float64)
    print(f"screened weights: median rel {np.median(rel):.2e}, max rel {rel.max():.2e}, "
          f"max dev/bound {float((dev / bound).max()):.3f}")
    assert np.median(rel) < 1e-6


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
    """Token 0, token T-1 and n-2 other random tokens (sorted, unique; all tokens when n >= T)."""
    if n >= T:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, T - 1), size=max(0, min(n - 2, T - 2)), replace=False) if T > 2 else []
    return np.array(sorted(set([0, T - 1]) | set(np.asarray(rest).tolist())))


def cover_tokens(idx: np.ndarray, offsets: np.ndarray, sorted_pair: np.ndarray, n_largest: int = 3,
                 tile: int = 256) -> np.ndarray:
    """Tokens whose outputs exercise every expert and every row tile of the largest experts.

    Greedy: tokens are added until every expert with rows has at least one of its
    (token, slot) pairs among them; then, for each of the n_largest experts, the
    tokens of the first and last row of every `tile`-row block of its rows (the GEMM
    row tiles, including the ragged last one); plus the first and last token."""
    T, k = idx.shape
    E = len(offsets) - 1
    need = set(np.nonzero(np.diff(offsets) > 0)[0].tolist())
    chosen = {0, T - 1}
    for t in (0, T - 1):
        need -= set(idx[t].tolist())
    for t in range(T):
        if not need:
            break
        new = need & set(idx[t].tolist())
        if new:
            chosen.add(t)
            need -= new
    counts = np.diff(offsets)
    for e in np.argsort(-counts, kind="stable")[:n_largest]:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(lo, hi, tile):
            for r in (r0, min(r0 + tile, hi) - 1):
                chosen.add(int(sorted_pair[r]) // k)
    return np.array(sorted(chosen))


def oracle_tokens(inp: G.MoEInputs, tokens: np.ndarray, routing, perm, workers: int = 16):
    """The oracle's outputs for `tokens` (routing and permutation given), computed over
    `workers` groups of tokens in a thread pool with one BLAS thread each; returns out
    [len(tokens), H] in the order of `tokens`.  Tokens are grouped so that each group
    touches few experts beyond the others' (the oracle dequantises every expert a
    group touches)."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    cfg = inp.cfg
    x = x_f64(inp)
    gw, b = inp.gate_w.double().cpu().numpy(), inp.bias.cpu().numpy()
    s13, s2 = shared_f64(inp)
    raw = expert_raw_fn(inp)
    idx = routing["idx"]
    nb = max(1, min(workers, len(tokens)))
    bins, sets = [[] for _ in range(nb)], [set() for _ in range(nb)]
    cap = -(-len(tokens) // nb)
    for t in tokens:                                    # greedy: fewest new experts, then emptiest group
        ex = set(idx[t].tolist())
        best = min((i for i in range(nb) if len(bins[i]) < cap), key=lambda i: (len(ex - sets[i]), len(sets[i])))
        bins[best].append(int(t))
        sets[best] |= ex

    def run(tk):
        return O.moe_forward(cfg, x, gw, b, raw, s13, s2, tokens=np.array(tk), routing=routing, perm=perm)["out"]

    with threadpool_limits(1), cf.ThreadPoolExecutor(max_workers=nb) as ex:
        outs = list(ex.map(run, [bn for bn in bins if bn]))
    got = dict(zip([t for bn in bins if bn for t in bn], np.concatenate(outs, axis=0)))
    return np.stack([got[int(t)] for t in tokens])


def row_rel_l2(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Relative L2 error of each row."""
    return np.linalg.norm(got - want, axis=1) / np.maximum(np.linalg.norm(want, axis=1), 1e-300)
