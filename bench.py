#!/usr/bin/env python3
"""Throughput of the block-scaled FP4 routed-expert MoE layer on one MI355X.

Headline: the decode-shaped layer (512 experts, top-10, hidden 2560, expert
intermediate 640, 16 tokens, NVFP4 weights with 4/6 block scales, bf16
activations): tokens/s of one moe_fp4_forward with inputs resident in HBM.
Weights are rotated over --copies resident copies of the quantized layer so
that successive steps cannot be served by the 256 MB Infinity Cache (a
48-layer model never re-reads one layer's experts back to back).

One JSON line: metric, value (tokens/s), ms_per_step, the roofline of the
dominant kernel (gate_up: algorithmic bytes / its average HIP-event duration
against 8 TB/s), per-stage times, and the CPU oracle timed on a bounded token
sample of the same workload.  Other workloads: --workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 MoE expert-layer tokens/s at B=16 and 8K; % of HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(cfg):
    """Bytes of one expert's gate_up and down weights in the layer's format."""
    H, I = cfg.hidden, cfg.inter
    n13, n2 = 2 * I * H, H * I
    if cfg.w_fmt == "nvfp4":
        return n13 // 2 + n13 // 16 + 4, n2 // 2 + n2 // 16 + 4
    if cfg.w_fmt == "mxfp4":
        return n13 // 2 + n13 // 32, n2 // 2 + n2 // 32
    return n13 + (2 * I // 128) * (H // 128) * 4, n2 + (H // 128) * (I // 128) * 4


def build_layer(cfg, torch, pkg):
    import numpy as np

    import synth
    t0 = time.perf_counter()
    w13, w2 = synth.layer_weights(cfg)
    log(f"generated bf16 weights in {time.perf_counter() - t0:.1f} s")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    g13 = up(w13)
    del w13
    q13 = pkg.quantize(g13, cfg.w_fmt, cfg.rule)
    del g13
    g2 = up(w2)
    del w2
    q2 = pkg.quantize(g2, cfg.w_fmt, cfg.rule)
    del g2
    torch.cuda.synchronize()
    return q13, q2


def make_layer(cfg, q13, q2, pkg):
    return pkg.MoELayer(cfg.w_fmt, cfg.a_fmt, cfg.num_experts, cfg.hidden, cfg.inter, cfg.top_k,
                        q13["codes"], q13["scales"], q2["codes"], q2["scales"],
                        q13.get("tensor_scale"), q2.get("tensor_scale"))


def clone_q(q):
    return {k: (v.clone() if v is not None else None) for k, v in q.items()}


def cpu_baseline(cfg, ids, wts, x_bits, budget_s=20.0):
    """The oracle (float64 numpy) on the first tokens of the same workload."""
    import numpy as np

    import synth
    from oracle import moe
    cores = len(os.sched_getaffinity(0))
    n = 1
    sample = list(range(n))
    touched = sorted({int(e) for t in sample for e in ids[t]})
    w13, w2 = synth.layer_weights(cfg, experts=touched)
    pos = {e: i for i, e in enumerate(touched)}
    q13 = {e: moe.quantize_expert_weight(w13[pos[e]], cfg.w_fmt, cfg.rule) for e in touched}
    q2 = {e: moe.quantize_expert_weight(w2[pos[e]], cfg.w_fmt, cfg.rule) for e in touched}
    layer = dict(w_fmt=cfg.w_fmt, a_fmt=cfg.a_fmt, num_experts=cfg.num_experts, hidden=cfg.hidden,
                 inter=cfg.inter, w13=lambda e: q13[e], w2=lambda e: q2[e])
    ids_s, wts_s, x_s = ids[:n], wts[:n], x_bits[:n]
    t0 = time.perf_counter()
    reps = 0
    while True:
        moe.moe_forward(layer, x_s, ids_s, wts_s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    tok_s = reps * n / el
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "threads_env": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{n} token(s) x {reps} repeat(s) of the {cfg.name} layer forward "
                      f"(dequantize-then-matmul in float64, weights pre-quantized by the oracle), "
                      f"{el:.1f} s"}


def bench_decode(args, torch, pkg):
    import numpy as np

    import synth
    cfg = synth.CONFIGS[args.workload]
    T = cfg.tokens
    q13, q2 = build_layer(cfg, torch, pkg)
    copies = [(q13, q2)] + [(clone_q(q13), clone_q(q2)) for _ in range(args.copies - 1)]
    layers = [make_layer(cfg, a, b, pkg) for a, b in copies]
    x_bits = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    tid = torch.from_numpy(ids).cuda()
    tw = torch.from_numpy(wts).cuda()
    ws = torch.empty(pkg.workspace_size(layers[0], T), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, cfg.hidden, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    for i in range(args.warmup):
        pkg.moe_forward(layers[i % len(layers)], x, tid, tw, ws, y)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        pkg.moe_forward(layers[i % len(layers)], x, tid, tw, ws, y)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps

    # per-stage durations (events recorded by the library between its launches)
    timer = pkg.StageTimer()
    acc = {s: 0.0 for s in pkg.STAGES}
    for i in range(args.steps):
        pkg.moe_forward_profiled(layers[i % len(layers)], x, tid, tw, ws, y, timer)
        torch.cuda.synchronize()
        for k, v in timer.durations().items():
            acc[k] += v
    stages = {k: v / args.steps for k, v in acc.items()}

    touched = len(np.unique(ids))
    b13, b2 = expert_bytes(cfg)
    P = T * cfg.top_k
    gateup_bytes = touched * b13 + T * cfg.hidden * 2 + P * cfg.inter * 4
    down_bytes = touched * b2 + P * cfg.inter * 4 + P * cfg.hidden * 4
    step_bytes = touched * (b13 + b2) + T * cfg.hidden * 2 + T * cfg.hidden * 4
    gu_ms = stages["gate_up"]
    roof = {"bound": "hbm", "kernel": "gemv_gateup_kernel",
            "achieved": gateup_bytes / (gu_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None,
            "bytes_per_launch": gateup_bytes,
            "unit_of_work": f"{touched} touched experts x {b13} B of NVFP4 gate_up weights"
                            f" + x {T * cfg.hidden * 2} B + h {P * cfg.inter * 4} B"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    out = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.num_experts} experts, top-{cfg.top_k}, hidden "
                               f"{cfg.hidden}, inter {cfg.inter}, {T} tokens, {cfg.w_fmt} "
                               f"({cfg.rule}) weights x bf16 activations",
                   "tokens": T, "touched_experts": int(touched), "layer_copies": len(layers)},
        "roofline": roof,
        "step_hbm": {"bytes": step_bytes, "GBps": step_bytes / (ms * 1e-3) / 1e9,
                     "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "stages_ms": stages,
        "down": {"bytes_per_launch": down_bytes,
                 "GBps": down_bytes / (stages["down"] * 1e-3) / 1e9 if stages["down"] > 0 else None},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, ids, wts, x_bits, args.cpu_budget)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode"])
    ap.add_argument("--copies", type=int, default=8,
                    help="resident copies of the quantized layer rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_fp4_nvfp4_amd as pkg
    pkg.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    out = bench_decode(args, torch, pkg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
