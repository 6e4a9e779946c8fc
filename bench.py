"""MoE-layer forward benchmark on one MI355X.

Times K calls of moe_forward (route, permute, grouped SwiGLU FFN, combine with the
shared expert) on seeded synthetic inputs already resident in HBM and prints one
JSON line.  The headline is the decode shape (T=128, H=7168, 384 experts, top-8,
I=2048, one shared expert, bf16):

- `value` / `ms_per_step`: K uninstrumented steps between two events on the
  launch stream;
- `roofline`: the dominant kernel (the routed gate/up GEMM step) from a second,
  instrumented pass of K steps in which the library records two HIP events around
  every launch on its stream;
- `configs`: the prefill shapes (bf16 grouped top-k, MXFP4, skewed fp8) measured
  the same way in the same run, each with its gate/up and routed-GEMM (gate/up +
  down) fractions of the binding peak -- HBM for the algorithmic bytes or MFMA for
  the flops, whichever takes longer at its peak, the other fraction beside it --
  and the layer's fraction of its roofline;
- `cpu_baseline`: the CPU oracle on the decode workload (see cpu_baseline()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {  # MI355X published dense peaks
    "hbm_GBps": 8000.0,
    "bf16_TFLOPs": 2516.6, "fp16_TFLOPs": 2516.6, "fp8_TFLOPs": 5033.2, "mxfp4_TFLOPs": 10066.3, "fp32_TFLOPs": 157.3,
}
EXTRA_CONFIGS = ("prefill_bf16_grouped", "finegrained_mxfp4", "skewed_fp8")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="decode_bf16")
    ap.add_argument("--extra-configs", default=",".join(EXTRA_CONFIGS),
                    help="comma-separated workloads also measured in this run ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=30.0,
                    help="seconds of single-core oracle FFN time before the rest is scaled from the experts done")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--residual", action="store_true",
                    help="time the residual form instead: out = h + MoE(RMSNorm(h)) (moe_forward_residual)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size reference for HBM counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def weight_bytes_per_element(recipe):
    """Stored bytes per weight element including scales, and activation bytes per element."""
    from workloads import configs as C
    return {C.RECIPE_BF16: (2.0, 2), C.RECIPE_F32: (4.0, 4), C.RECIPE_FP8_B128: (1.0 + 4.0 / (128 * 128), 1),
            C.RECIPE_NVFP4: (0.5 + 1.0 / 16, 2), C.RECIPE_MXFP4: (0.5 + 1.0 / 32, 1)}[recipe]


def mfma_peak(recipe):
    from workloads import configs as C
    return PEAK[{C.RECIPE_BF16: "bf16_TFLOPs", C.RECIPE_FP8_B128: "fp8_TFLOPs", C.RECIPE_MXFP4: "fp8_TFLOPs",
                 C.RECIPE_F32: "fp32_TFLOPs", C.RECIPE_NVFP4: "fp16_TFLOPs"}[recipe]]


def gate_up_work(cfg, touched):
    """Algorithmic work of one launch of the routed gate/up step (a7): per touched
    expert its gate_proj + up_proj weights (2*I*H elements + scales) streamed once; per
    pair row the activation row read (H) and the h row written (I).  FLOPs:
    2 * (T*k) * H * 2I."""
    I, H, P = cfg.intermediate, cfg.hidden, cfg.pairs
    wb, ab = weight_bytes_per_element(cfg.recipe)
    bytes_ = touched * 2 * I * H * wb + P * H * ab + P * I * ab
    return bytes_, 2.0 * P * H * 2 * I


def routed_work(cfg, touched):
    """Routed gate/up + down (a7 + a8): touched experts' 3*I*H weights (+ scales) once;
    FLOPs 2 * (T*k) * 3 * H * I."""
    I, H, P = cfg.intermediate, cfg.hidden, cfg.pairs
    wb, _ = weight_bytes_per_element(cfg.recipe)
    return touched * 3 * I * H * wb, 2.0 * P * 3 * H * I


def layer_roofline_tokens_per_s(cfg, touched):
    """T over the larger of the MFMA time (each precision at its peak, the gate at the
    fp32 rate the method specifies) and the HBM time of the algorithmic bytes (touched
    experts' weights and scales, shared and gate weights, x read, out written)."""
    from workloads import configs as C
    T, H, I, E = cfg.num_tokens, cfg.hidden, cfg.intermediate, cfg.num_experts
    SI = cfg.num_shared * cfg.shared_intermediate
    w_bytes, r_flops = routed_work(cfg, touched)
    sh_b = 4 if cfg.recipe == C.RECIPE_F32 else 2
    t_mfma = (r_flops / mfma_peak(cfg.recipe) + 6.0 * T * H * SI / (PEAK["fp32_TFLOPs"] if sh_b == 4 else PEAK["bf16_TFLOPs"])
              + 2.0 * T * H * E / PEAK["fp32_TFLOPs"]) / 1e12
    bytes_ = w_bytes + 3 * H * SI * sh_b + E * H * 4 + 2 * T * H * sh_b
    t_hbm = bytes_ / (PEAK["hbm_GBps"] * 1e9)
    return T / max(t_mfma, t_hbm)


def traffic_from_profiles(cfg_name: str, src_hash: str):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter
    runs, or None when absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_ffn_gate_up_{cfg_name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


def run_workload(cfg, args, residual=False):
    """Generate the workload on the GPU, time K uninstrumented steps, then K
    instrumented ones.  Returns (inputs, buffers, ms per step, per-kernel ms/launches)."""
    import torch

    import mixture_experts_amd as M
    from workloads import generate as G

    t_gen = time.time()
    inp = G.generate(cfg, device="cuda")
    mcfg = M.make_config(cfg)
    b = M.alloc_buffers(mcfg, "cuda")
    ex = M.make_expert_weights(cfg.recipe, inp.w13, inp.w2, inp.w13_scale, inp.w2_scale)   # fp4: scales packed once
    sh = M.make_weights(inp.shared_w13, inp.shared_w2) if cfg.num_shared > 0 else None
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: inputs ready in {time.time() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def step():
        if residual:
            M.moe_forward_residual(mcfg, inp.x, inp.norm_w, G.RMS_EPS, inp.gate_w, inp.bias, ex, sh, b.out,
                                   b.topk_idx, b.topk_w, b.ws)
        else:
            M.moe_forward(mcfg, inp.x, inp.gate_w, inp.bias, ex, sh, b.out, b.topk_idx, b.topk_w, b.ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()          # the stream the library launches on
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    # the per-kernel breakdown: the same steps again, every launch between two events
    M.moe_profile_start(64 * (args.steps + 1))
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        step()
    f1.record(stream)
    torch.cuda.synchronize()
    prof = M.moe_profile_stop()
    ms_step_instr = f0.elapsed_time(f1) / args.steps
    print(f"[bench] {cfg.name}: {ms_step:.3f} ms/step ({ms_step_instr:.3f} instrumented)", file=sys.stderr, flush=True)
    return inp, b, ms_step, ms_step_instr, prof


def _bound(bytes_, flops, t_s, recipe):
    """The binding roofline of a step: HBM (algorithmic bytes) or MFMA (flops), whichever
    takes longer at its peak; the other one's fraction is reported beside it."""
    pk = mfma_peak(recipe)
    hbm = {"bound": "hbm", "achieved": bytes_ / t_s / 1e9, "peak": PEAK["hbm_GBps"], "unit": "GB/s"}
    mf = {"bound": "mfma", "achieved": flops / t_s / 1e12, "peak": pk, "unit": "TFLOP/s"}
    for d in (hbm, mf):
        d["achieved"] = round(d["achieved"], 1)
        d["frac"] = round(d["achieved"] / d["peak"], 4)
    t_hbm, t_mf = bytes_ / (PEAK["hbm_GBps"] * 1e9), flops / (pk * 1e12)
    main, other = (hbm, mf) if t_hbm >= t_mf else (mf, hbm)
    main["roofline_ms"] = round(max(t_hbm, t_mf) * 1e3, 4)
    main["other"] = other
    return main


def fractions(cfg, counts, prof, steps):
    """Gate/up and routed (gate/up + down) fractions of the binding peak."""
    touched = int((counts > 0).sum())
    ms_gu, n_gu = prof["ffn_gate_up"]
    ms_dn, n_dn = prof["ffn_down"]
    avg_gu = ms_gu / max(n_gu, 1)
    gu_bytes, gu_flops = gate_up_work(cfg, touched)
    r_bytes, r_flops = routed_work(cfg, touched)
    t_routed = (ms_gu + ms_dn) / steps * 1e-3
    gu = _bound(gu_bytes, gu_flops, avg_gu * 1e-3, cfg.recipe)
    rt = _bound(r_bytes, r_flops, t_routed, cfg.recipe)
    gu["avg_launch_ms"] = round(avg_gu, 4)
    gu["algorithmic_per_launch"] = gu_bytes if gu["bound"] == "hbm" else gu_flops
    rt["ms_per_step"] = round(t_routed * 1e3, 4)
    return touched, gu, rt


def cpu_baseline(cfg, inp, budget_s):
    """The oracle (numpy fp64, as it stands) on the whole workload, timed on the host.
    Routing and permutation of all T tokens and the shared expert(s) over all T tokens
    are timed in full.  The routed FFN -- per touched expert: dequantise its weights,
    run its MLP on all of its rows -- is timed expert by expert in a seeded random
    order until every touched expert is done or budget_s has passed; in the second
    case the time is scaled to all touched experts (the sample says which).
    Primary figure: one core (BLAS and every step on one thread).  Secondary: all
    host cores (up to 16 threads, one BLAS thread each, over all touched experts)."""
    import concurrent.futures as cf

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as O
    from tests import harness as HN
    T, I, H = cfg.num_tokens, cfg.intermediate, cfg.hidden
    quant = cfg.recipe in (O.RECIPE_FP8_B128, O.RECIPE_MXFP4, O.RECIPE_NVFP4)
    # host copies of the inputs (not timed: I/O, not oracle work)
    x64 = HN.x_f64(inp)
    gw = inp.gate_w.double().cpu().numpy()
    bias = inp.bias.cpu().numpy()
    s13, s2 = HN.shared_f64(inp)
    raw_fn = HN.expert_raw_fn(inp)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        routing = O.route(cfg, x64, gw, bias)
        O.permute(routing["idx"], cfg.num_experts)
        t_route = time.perf_counter() - t0
    idx = routing["idx"]
    touched = np.random.default_rng(1).permutation(np.unique(idx))
    raw = {int(e): raw_fn(int(e)) for e in touched}
    xq = O.quantize_rows(cfg.recipe, x64.astype(np.float32)) if quant else x64

    def one_expert(e):                                   # moe_forward's per-expert step
        rows, _ = np.nonzero(idx == e)
        w13, w2 = O.dequant_expert(cfg.recipe, raw[int(e)], I, H)
        return O.expert_mlp(xq[rows], w13, w2, cfg.recipe, quantize_h=quant)

    with threadpool_limits(1):
        done, t0 = 0, time.perf_counter()
        for e in touched:
            one_expert(e)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        t_ffn = time.perf_counter() - t0
        t0 = time.perf_counter()
        for s in range(s13.shape[0]):
            O.expert_mlp(x64, s13[s], s2[s])
        t_shared = time.perf_counter() - t0
    t1 = t_route + t_shared + t_ffn / done * touched.size
    ncpu = os.cpu_count() or 1
    workers = min(ncpu, 16)
    with threadpool_limits(1), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        t0 = time.perf_counter()
        list(ex.map(one_expert, touched))
        t_ffn_mt = time.perf_counter() - t0
    with threadpool_limits(workers):
        t0 = time.perf_counter()
        for s in range(s13.shape[0]):
            O.expert_mlp(x64, s13[s], s2[s])
        t_shared_mt = time.perf_counter() - t0
    tn = t_route + t_shared_mt + t_ffn_mt
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass
    ffn = (f"the routed FFN of all {touched.size} touched experts ({t_ffn:.1f} s)" if done == touched.size else
           f"the routed FFN timed on {done} of the {touched.size} touched experts (all their rows; {t_ffn:.1f} s) "
           f"and scaled to all of them")
    return {"value": round(T / t1, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload, all {T} tokens, on one core: routing + permutation and the shared "
                      f"expert ({t_route + t_shared:.1f} s), {ffn}; {t1:.1f} s in all",
            "all_cores": {"value": round(T / tn, 4), "threads": workers, "seconds": round(tn, 2)},
            "nproc": ncpu, "cpu_model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the layer's multi-GPU "
              f"expert-parallel path is not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from workloads import configs as C

    cfg = C.get(args.config)
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)                  # one elementwise kernel: reads and writes N MiB
        torch.cuda.synchronize()
        del src, dst
    w0 = time.perf_counter()
    inp, b, ms_step, ms_instr, prof = run_workload(cfg, args, residual=args.residual)
    wall = time.perf_counter() - w0
    value = cfg.num_tokens / (ms_step / 1e3)
    counts = np.bincount(b.topk_idx.cpu().numpy().reshape(-1), minlength=cfg.num_experts)
    touched, gu, rt = fractions(cfg, counts, prof, args.steps)
    src_hash = kernel_source_hash()
    roof = {k: gu[k] for k in ("bound", "achieved", "peak", "unit", "frac", "roofline_ms", "other")}
    roof["traffic"] = traffic_from_profiles(cfg.name, src_hash)
    roof.update(kernel="ffn_gate_up", avg_launch_ms=gu["avg_launch_ms"],
                algorithmic_per_launch=gu["algorithmic_per_launch"], routed_gate_up_down=rt)
    roof_tps = layer_roofline_tokens_per_s(cfg, touched)

    dtype = {C.RECIPE_F32: "f32", C.RECIPE_BF16: "bf16", C.RECIPE_FP8_B128: "fp8_e4m3",
             C.RECIPE_MXFP4: "mxfp4xmxfp8", C.RECIPE_NVFP4: "nvfp4 (fp16 MFMA)"}[cfg.recipe]
    line = {
        "metric": "MoE-layer tokens/s (one layer forward, 1 GPU)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": cfg.name, "T": cfg.num_tokens, "H": cfg.hidden, "E": cfg.num_experts,
                   "top_k": cfg.top_k, "I": cfg.intermediate, "shared": cfg.num_shared,
                   "shared_I": cfg.shared_intermediate, "n_group": cfg.n_group, "topk_group": cfg.topk_group,
                   "recipe": C.RECIPE_NAMES[cfg.recipe], "touched_experts": touched,
                   "max_expert_rows": int(counts.max()), "parallelism": "single GPU",
                   "form": "residual (h + MoE(RMSNorm(h)))" if args.residual else "moe"},
        "roofline": roof,
        "layer_roofline": {"tokens_per_s": round(roof_tps, 1), "frac": round(value / roof_tps, 4)},
        "ms_per_step_instrumented": round(ms_instr, 4),
        "kernels_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in prof.items() if v[1]},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
        print(f"[bench] cpu baseline in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        if args.residual:
            line["cpu_baseline"]["sample"] += " (MoE part of the residual form)"
    del inp, b
    torch.cuda.empty_cache()
    extra = {}
    for name in [n for n in args.extra_configs.split(",") if n and n != cfg.name]:
        c2 = C.get(name)
        inp2, b2, ms2, ms2i, prof2 = run_workload(c2, args)
        counts2 = np.bincount(b2.topk_idx.cpu().numpy().reshape(-1), minlength=c2.num_experts)
        t2, gu2, rt2 = fractions(c2, counts2, prof2, args.steps)
        tps = c2.num_tokens / (ms2 / 1e3)
        rtps = layer_roofline_tokens_per_s(c2, t2)
        gu2["traffic"] = traffic_from_profiles(c2.name, src_hash)
        extra[name] = {"T": c2.num_tokens, "recipe": C.RECIPE_NAMES[c2.recipe], "ms_per_step": round(ms2, 4),
                       "tokens_per_s": round(tps, 1), "layer_roofline_tokens_per_s": round(rtps, 1),
                       "layer_frac": round(tps / rtps, 4), "touched_experts": t2,
                       "max_expert_rows": int(counts2.max()), "gate_up": gu2, "routed_gate_up_down": rt2,
                       "ms_per_step_instrumented": round(ms2i, 4),
                       "kernels_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in prof2.items() if v[1]}}
        del inp2, b2
        torch.cuda.empty_cache()
    if extra:
        line["configs"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
