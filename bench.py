"""MoE-layer forward benchmark on one MI355X.

Times K calls of moe_forward (route, permute, grouped SwiGLU FFN, combine with the
shared expert) on seeded synthetic inputs already resident in HBM, and prints one
JSON line: tokens/s, the dominant kernel's roofline fraction (per-launch durations
from HIP events recorded on the launch stream by the library's instrumentation),
and the CPU oracle timed on a bounded sample of the same workload.

Default workload: the decode shape (T=128, H=7168, 384 experts, top-8, I=2048,
one shared expert, bf16).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {  # MI355X published peaks (dense)
    "hbm_GBps": 8000.0,
    "bf16_TFLOPs": 2516.6, "fp16_TFLOPs": 2516.6, "fp8_TFLOPs": 5033.2, "mxfp4_TFLOPs": 10066.3, "fp32_TFLOPs": 157.3,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="decode_bf16")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens in the oracle's timed sample")
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


def dominant_kernel_work(cfg, counts):
    """Algorithmic work of one launch of the routed gate/up grouped GEMM (the dominant kernel).

    Per touched expert: its gate_proj + up_proj weights (2*I*H elements + scales) are
    streamed once; per pair row: x_perm row read (H) and h row written (I).
    FLOPs: 2 * (T*k) * H * 2I."""
    from workloads import configs as C
    I, H, P = cfg.intermediate, cfg.hidden, cfg.pairs
    touched = int((counts > 0).sum())
    n = 2 * I * H
    if cfg.recipe == C.RECIPE_BF16:
        wbytes, abytes = 2 * n, 2
    elif cfg.recipe == C.RECIPE_F32:
        wbytes, abytes = 4 * n, 4
    elif cfg.recipe == C.RECIPE_FP8_B128:
        wbytes, abytes = n + 4 * n // (128 * 128), 1
    elif cfg.recipe == C.RECIPE_NVFP4:
        wbytes, abytes = n // 2 + n // 16, 2
    else:
        wbytes, abytes = n // 2 + n // 32, 1
    bytes_ = touched * wbytes + P * H * abytes + P * I * abytes
    flops = 2.0 * P * H * 2 * I
    return touched, bytes_, flops, wbytes


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


def cpu_baseline(cfg, inp, n_sample):
    """The oracle (numpy fp64, as it stands) on a bounded sample: routing of every
    token plus the expert and shared MLPs of n_sample tokens."""
    import numpy as np
    from oracle import moe_oracle as O
    from tests import harness as HN
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    tokens = HN.sample_tokens(cfg.num_tokens, n_sample, seed=1)
    # host copies of the inputs (not timed: this is I/O, not oracle work)
    x64 = HN.x_f64(inp)
    gw = inp.gate_w.double().cpu().numpy()
    bias = inp.bias.cpu().numpy()
    s13, s2 = HN.shared_f64(inp)
    routing = O.route(cfg, x64, gw, bias)
    experts = sorted(set(routing["idx"][tokens].reshape(-1).tolist()))
    raw_fn = HN.expert_raw_fn(inp)
    raw = {e: raw_fn(e) for e in experts}
    t0 = time.perf_counter()
    O.moe_forward(cfg, x64, gw, bias, lambda e: raw[e], s13, s2, tokens=tokens)
    dt = time.perf_counter() - t0
    return {"value": round(len(tokens) / dt, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(tokens)} of {cfg.num_tokens} tokens ({len(experts)} distinct experts); routing of all "
                      f"{cfg.num_tokens} tokens included; {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the layer's multi-GPU "
              f"expert-parallel path is not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_amd as M
    from workloads import configs as C
    from workloads import generate as G

    cfg = C.get(args.config)
    torch.cuda.set_device(0)
    t_gen = time.time()
    inp = G.generate(cfg, device="cuda")
    mcfg = M.make_config(cfg)
    b = M.alloc_buffers(mcfg, "cuda")
    ex = M.make_expert_weights(cfg.recipe, inp.w13, inp.w2, inp.w13_scale, inp.w2_scale)   # fp4: scales packed once
    sh = M.make_weights(inp.shared_w13, inp.shared_w2) if cfg.num_shared > 0 else None
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: inputs ready in {time.time() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def step():
        if args.residual:
            M.moe_forward_residual(mcfg, inp.x, inp.norm_w, G.RMS_EPS, inp.gate_w, inp.bias, ex, sh, b.out,
                                   b.topk_idx, b.topk_w, b.ws)
        else:
            M.moe_forward(mcfg, inp.x, inp.gate_w, inp.bias, ex, sh, b.out, b.topk_idx, b.topk_w, b.ws)

    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)                  # one elementwise kernel: reads and writes N MiB
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    M.moe_profile_start(64 * (args.steps + 1))
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    prof = M.moe_profile_stop()
    ms_step = e0.elapsed_time(e1) / args.steps
    value = cfg.num_tokens / (ms_step / 1e3)

    counts = np.bincount(b.topk_idx.cpu().numpy().reshape(-1), minlength=cfg.num_experts)
    touched, kbytes, kflops, wbytes = dominant_kernel_work(cfg, counts)
    ms_k, n_k = prof["ffn_gate_up"]
    avg_k = ms_k / max(n_k, 1)
    hbm_bound = cfg.name in ("decode_bf16", "finegrained_mxfp4", "tiny_fp32", "decode_nvfp4")
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles(cfg.name, src_hash)
    if hbm_bound:
        achieved = kbytes / (avg_k * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_GBps"], "unit": "GB/s"}
    else:
        pk = {C.RECIPE_BF16: "bf16_TFLOPs", C.RECIPE_FP8_B128: "fp8_TFLOPs", C.RECIPE_MXFP4: "mxfp4_TFLOPs",
              C.RECIPE_F32: "fp32_TFLOPs", C.RECIPE_NVFP4: "fp16_TFLOPs"}[cfg.recipe]
        achieved = kflops / (avg_k * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK[pk], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic
    roof["kernel"] = "ffn_gate_up"
    roof["avg_launch_ms"] = round(avg_k, 4)
    roof["algorithmic_per_launch"] = kbytes if hbm_bound else kflops

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
        "kernels_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in prof.items() if v[1]},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        n = args.cpu_sample or {"tiny_fp32": 64, "decode_bf16": 6, "prefill_bf16_grouped": 6,
                                "finegrained_mxfp4": 4, "skewed_fp8": 6}.get(cfg.name, 8)
        line["cpu_baseline"] = cpu_baseline(cfg, inp, n)
        if args.residual:
            line["cpu_baseline"]["sample"] += " (MoE part of the residual form)"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
