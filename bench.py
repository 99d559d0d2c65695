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
sample of the same workload.  The other workloads of the layer (8192-token
prefill in NVFP4 W4A4 with the MXFP8 shared expert, MXFP4 x MXFP8, block FP8,
and the 48-layer streaming 4/6 quantization) are reported in the same line
under "workloads", each with its own roofline and oracle baseline.
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


def make_layer(cfg, q13, q2, pkg, shared=None):
    layer = pkg.MoELayer(cfg.w_fmt, cfg.a_fmt, cfg.num_experts, cfg.hidden, cfg.inter, cfg.top_k,
                         q13["codes"], q13["scales"], q2["codes"], q2["scales"],
                         q13.get("tensor_scale"), q2.get("tensor_scale"))
    if shared is not None:
        a, b, gate = shared
        layer.shared_inter = cfg.shared_inter
        layer.ws13, layer.ws13_scale = a["codes"], a["scales"]
        layer.ws2, layer.ws2_scale = b["codes"], b["scales"]
        layer.shared_gate = gate
    return layer


def build_shared(cfg, torch, pkg):
    import numpy as np

    import synth
    s13, s2, gate = synth.shared_expert(cfg)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return pkg.quantize(up(s13), "mxfp8"), pkg.quantize(up(s2), "mxfp8"), up(gate)


def clone_q(q):
    return {k: (v.clone() if v is not None else None) for k, v in q.items()}


def cpu_baseline(cfg, ids, wts, x_bits, budget_s=20.0):
    """The oracle (float64 numpy) on the first token of the same workload (for
    NVFP4 activations the tensor scales then come from that token's rows)."""
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
    layer = dict(w_fmt=cfg.w_fmt, a_fmt=cfg.a_fmt,
                 num_experts=cfg.num_experts, hidden=cfg.hidden,
                 inter=cfg.inter, w13=lambda e: q13[e], w2=lambda e: q2[e])
    if cfg.shared_inter:
        s13, s2, gate = synth.shared_expert(cfg)
        layer["shared"] = dict(w13=moe.quantize_expert_weight(s13, "mxfp8"),
                               w2=moe.quantize_expert_weight(s2, "mxfp8"), gate_bits=gate)
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


def time_route(cfg, torch, pkg, reps=50):
    """GPU top-k routing (moe_fp4_route) of the workload's router logits: the
    caller-side step in front of the layer, timed on its own (it is not part
    of the layer step above)."""
    import numpy as np

    import synth
    lg = torch.from_numpy(synth.router_logits(cfg)).cuda()
    bias = torch.from_numpy(synth.router_bias(cfg)).cuda() if cfg.router_bias else None
    for _ in range(3):
        pkg.route(lg, cfg.top_k, bias)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        pkg.route(lg, cfg.top_k, bias)
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) / reps * 1e3
    ids, _ = pkg.route(lg, cfg.top_k, bias)
    same = bool(np.array_equal(ids.cpu().numpy(), synth.routing(cfg)[0]))
    return {"us_per_call": us, "tokens": cfg.tokens, "experts": cfg.num_experts, "k": cfg.top_k,
            "biased": bool(cfg.router_bias), "ids_equal_host_routing": same}


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
    tr = measured_traffic("gemv_gateup_kernel", "decode")
    roof = {"bound": "hbm", "kernel": "gemv_gateup_kernel",
            "achieved": gateup_bytes / (gu_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": tr["bytes_per_launch"] if tr else None,
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
        "route": time_route(cfg, torch, pkg),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, ids, wts, x_bits, args.cpu_budget)
    return out


def time_steps(pkg, torch, layers, x, tid, tw, ws, y, steps, warmup):
    for i in range(warmup):
        pkg.moe_forward(layers[i % len(layers)], x, tid, tw, ws, y)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        pkg.moe_forward(layers[i % len(layers)], x, tid, tw, ws, y)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    timer = pkg.StageTimer()
    acc = {s_: 0.0 for s_ in pkg.STAGES}
    for i in range(steps):
        pkg.moe_forward_profiled(layers[i % len(layers)], x, tid, tw, ws, y, timer)
        torch.cuda.synchronize()
        for k_, v in timer.durations().items():
            acc[k_] += v
    return ms, {k_: v / steps for k_, v in acc.items()}


def bench_prefill(name, args, torch, pkg):
    import numpy as np

    import synth
    cfg = synth.CONFIGS[name]
    T, P, H, I = cfg.tokens, cfg.pairs, cfg.hidden, cfg.inter
    q13, q2 = build_layer(cfg, torch, pkg)
    shared = build_shared(cfg, torch, pkg) if cfg.shared_inter else None
    layers = [make_layer(cfg, q13, q2, pkg, shared)]
    for _ in range(max(0, args.prefill_copies - 1)):
        layers.append(make_layer(cfg, clone_q(q13), clone_q(q2), pkg, shared))
    tiled = args.weight_layout == "tiled"
    if tiled:  # once per layer, like its quantization: outside the timed region
        for layer in layers:
            layer.w13_tiled, layer.w13_scale_tiled = pkg.tile_weights(layer.w13, layer.w13_scale, cfg.w_fmt)
            layer.w2_tiled, layer.w2_scale_tiled = pkg.tile_weights(layer.w2, layer.w2_scale, cfg.w_fmt)
        torch.cuda.synchronize()
    x_bits = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    tid, tw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    ws = torch.empty(pkg.workspace_size(layers[0], T), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.float32, device="cuda")
    ms, stages = time_steps(pkg, torch, layers, x, tid, tw, ws, y, args.prefill_steps, 2)
    flops_gu = 4.0 * P * H * I
    flops_down = 2.0 * P * H * I
    flops_shared = 6.0 * T * H * cfg.shared_inter
    counts = np.bincount(ids.reshape(-1), minlength=cfg.num_experts)
    touched = int((counts > 0).sum())
    b13, b2 = expert_bytes(cfg)
    weight_bytes = touched * (b13 + b2)
    peak_key = "bf16" if cfg.a_fmt == "nvfp4" else "fp8"
    peak = MFMA_PEAK_TFLOPS[peak_key]
    gu_ms = stages["gate_up"]
    roof = {"bound": "mfma", "kernel": "grouped_gemm_kernel (gate_up)", "mfma_dtype":
            {"bf16": "fp16 (exact NVFP4 decode)", "fp8": "fp8 x fp4" if cfg.w_fmt == "mxfp4" else "fp8"}[peak_key],
            "achieved": flops_gu / (gu_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
            "traffic": (lambda t: t["bytes_per_launch"] if t else None)(
                measured_traffic("grouped_gemm_kernel_gateup", name)),
            "flops_per_launch": flops_gu,
            "unit_of_work": f"{P} (token, expert) rows x 2 x {2 * I} x {H} FLOPs"}
    roof["frac"] = roof["achieved"] / peak
    total_flops = flops_gu + flops_down + flops_shared
    out = {"workload": f"{cfg.name}: {cfg.num_experts} experts, top-{cfg.top_k}, hidden {H}, inter {I}, "
                       f"{T} tokens, {cfg.w_fmt} weights x {cfg.a_fmt} activations"
                       + (f", MXFP8 shared expert {cfg.shared_inter}" if cfg.shared_inter else "")
                       + (", W13 and W2 tiled for the GEMMs" if tiled else ""),
           "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "steps": args.prefill_steps,
           "dtype": {"nvfp4": "fp16", "mxfp8": "fp8", "fp8_row": "fp8"}[cfg.a_fmt],
           "roofline": roof, "stages_ms": stages,
           "step_mfma": {"flops": total_flops, "TFLOPs": total_flops / (ms * 1e-3) / 1e12,
                         "frac_of_peak": total_flops / (ms * 1e-3) / 1e12 / peak},
           "step_hbm": {"weight_bytes": weight_bytes, "touched_experts": touched,
                        "max_rows_per_expert": int(counts.max())},
           "route": time_route(cfg, torch, pkg, reps=20)}
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {name}")
        out["cpu_baseline"] = cpu_baseline(cfg, ids, wts, x_bits, args.cpu_budget)
    del layers, q13, q2
    torch.cuda.empty_cache()
    return out


def file_sha(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by what the
    same counters read for a plain copy of known size), or None when the
    summary is absent or the kernel's source file changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or "=" not in line:
            continue
        kv = dict(t.split("=", 1) for t in line.split())
        if kv.get("kernel") != kernel or kv.get("workload") != workload:
            continue
        if file_sha(kv["source"]) != kv["source_sha"]:
            return None
        return {"bytes_per_launch": float(kv["bytes_per_launch"]), "fetch_bytes": float(kv["fetch_bytes"]),
                "write_bytes": float(kv["write_bytes"]), "copy_scale": float(kv["copy_scale"]),
                "source": kv["source"]}
    return None


def bench_copy(args, torch):
    """A plain device copy (elementwise negation of 2^28 float32 values: one
    1 GiB read and one 1 GiB write per launch), used to calibrate the HBM byte
    counters against a kernel of known traffic."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        torch.neg(a, out=b)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    return {"metric": "plain copy GB/s", "value": 2 * n * 4 / (ms * 1e-3) / 1e9, "unit": "GB/s",
            "bytes_read": n * 4, "bytes_written": n * 4, "ms_per_launch": ms, "steps": args.steps}


def bench_stream_quant(args, torch, pkg, rule="4over6"):
    """48 layers x 512 experts x (gate_up 1280x2560, down 2560x640) NVFP4
    quantization (4/6, or the scale sweep), one layer at a time, from bf16
    Student-t (nu=4) source with 1% outlier rows x8 generated on the device
    for each layer.  The sweep workload also reports, on its first and last
    layer, the 4/6 error of the same tensors."""
    import numpy as np
    E, H, I = 512, 2560, 640
    layers = args.stream_layers if rule == "4over6" else args.sweep_layers
    gen = torch.Generator(device="cuda")
    tdist = torch.distributions.StudentT(torch.tensor(4.0, device="cuda"))

    def source(layer, rows, cols):
        gen.manual_seed(1000 + layer * 7 + rows)
        torch.manual_seed(2000 + layer * 7 + rows)
        v = tdist.sample((E, rows, cols)) * (0.02 / 2 ** 0.5)
        n_out = int(round(0.01 * rows))
        idx = torch.argsort(torch.rand(E, rows, device="cuda", generator=gen), dim=1)[:, :n_out]
        v.scatter_(1, idx[:, :, None].expand(E, n_out, cols), v.gather(1, idx[:, :, None].expand(E, n_out, cols)) * 8)
        return v.to(torch.bfloat16)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_ms = 0.0
    stats = []
    rd = wr = 0
    for layer in range(layers):
        w13 = source(layer, 2 * I, H)
        w2 = source(layer, H, I)
        torch.cuda.synchronize()
        want = layer in (0, layers - 1) and not args.no_quality
        start.record()
        q13 = pkg.quantize(w13, "nvfp4", rule, want_m4=want)
        q2 = pkg.quantize(w2, "nvfp4", rule, want_m4=want)
        stop.record()
        torch.cuda.synchronize()
        total_ms += start.elapsed_time(stop)
        for w, q in ((w13, q13), (w2, q2)):
            rd += w.numel() * 2
            wr += q["codes"].numel() + q["scales"].numel() + q["tensor_scale"].numel() * 4
        if want:
            for w, q, names in ((w13, q13, ("gate", "up")), (w2, q2, ("down",))):
                # squared error of every block from the library (fp4_block_error)
                be = pkg.block_error(w, q, "nvfp4").double()
                src = w.double()
                parts = [(n, sl) for n, sl in zip(names, (slice(0, I), slice(I, 2 * I)))] if len(names) == 2 \
                    else [("down", slice(0, H))]
                be46 = None
                if rule != "4over6":  # the same tensors under 4/6, for comparison (untimed)
                    be46 = pkg.block_error(w, pkg.quantize(w, "nvfp4", "4over6"), "nvfp4").double()
                for n, sl in parts:
                    d = be[:, sl].sum(dim=(1, 2))
                    nrm = src[:, sl].pow(2).sum(dim=(1, 2))
                    rel = (d / nrm).sqrt()
                    rel46 = None
                    if be46 is not None:
                        rel46 = float((be46[:, sl].sum(dim=(1, 2)) / nrm).sqrt().mean())
                    stats.append((n, float(rel.mean()), float(rel.max()),
                                  float((q["m4"][:, sl] > 0).float().mean()), float(d.sum()), float(nrm.sum()),
                                  rel46))
                del be, src, be46
        del w13, w2, q13, q2
    ms_layer = total_ms / layers
    bytes_layer = (rd + wr) / layers
    gbs = bytes_layer / (ms_layer * 1e-3) / 1e9
    rule_name = {"4over6": "4/6", "sweep": "scale-sweep"}[rule]
    out = {"workload": f"streaming NVFP4 {rule_name} quantization: {layers} layers x {E} experts x "
                       f"(gate_up {2 * I}x{H}, down {H}x{I}), bf16 Student-t(4) source with 1% outlier rows x8",
           "value": gbs, "unit": "GB/s", "ms_per_layer": ms_layer, "layers": layers,
           "values_per_layer": E * 3 * H * I,
           "roofline": {"bound": "hbm", "kernel": "quant_fp4_kernel (fused with the next chunk's amax) + tensor_amax_kernel (first chunk)",
                        "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "traffic": (lambda t: t["bytes_per_launch"] if t else None)(
                            measured_traffic("quant_fp4_kernel", "stream_quant" if rule == "4over6" else "sweep_quant")),
                        "bytes_per_layer": bytes_layer,
                        "unit_of_work": "2 B read + 0.5625 B written per value (+4 B per tensor)"},
           "quality": {"per_tensor_rel_err": {n: {"mean": m, "max": mx} for n, m, mx, *_ in stats},
                       "m4_fraction": float(np.mean([st[3] for st in stats])) if stats else None}}
    if rule != "4over6" and stats:
        out["quality"]["per_tensor_rel_err_4over6_same_data"] = {st[0]: {"mean": st[6]} for st in stats}
        out["quality"]["note"] = ("m4_fraction: blocks whose scale is not the amax/6 plan's; "
                                  "first and last layer")
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on streaming quantization ({rule})")
        import synth
        from oracle import quant
        from oracle.formats import bf16_to_f64
        t0 = time.perf_counter()
        n_vals = 0
        e = 0
        budget = args.cpu_budget if rule == "4over6" else args.cpu_budget / 2
        while time.perf_counter() - t0 < budget and e < 64:
            w13, w2 = synth.streaming_expert(0, e)
            for w in (w13, w2):
                quant.quantize_nvfp4(bf16_to_f64(w), rule)
                n_vals += w.size
            e += 1
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n_vals * 2.5625 / el / 1e9, "unit": "GB/s", "values_per_s": n_vals / el,
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"{e} expert(s) of layer 0 (gate_up + down), source drawn on the host, "
                                         f"{el:.1f} s"}
    return out


def bench_stack(args, torch, pkg):
    """Decode of 16 tokens through the 48-layer mixed-precision routed-expert
    stack of the MXFP4-FP8-R12 card (layers 19, 20, 21, 23, 28, 32, 33, 40,
    41, 43, 44, 45 block FP8 x dynamic FP8, the other 36 MXFP4 x dynamic
    MXFP8; 512 experts, top-10, hidden 2560, inter 640), all 48 layers resident
    (78.3 GB of expert weights; the block-FP8 layers also hold the tiled
    copies their GEMMs read) and run as one captured HIP graph per step.
    Weights N(0, 0.02) bf16 drawn on the device per layer and quantized by the
    library; each layer gets its own synthetic tokens and routing."""
    import numpy as np

    import synth
    from block_scaled_fp4_nvfp4_amd.stack import LayerStack
    cfgs = synth.stack_configs(n_layers=args.stack_layers)
    gen = torch.Generator(device="cuda")
    layers, xs, ids_l, ws_l, touched, wbytes = [], [], [], [], [], 0
    t0 = time.perf_counter()
    for cfg in cfgs:
        qs = []
        for proj, rows, cols in ((0, 2 * cfg.inter, cfg.hidden), (1, cfg.hidden, cfg.inter)):
            gen.manual_seed(cfg.weight_seed * 10 + proj)
            w = (torch.randn(cfg.num_experts, rows, cols, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
            qs.append(pkg.quantize(w, cfg.w_fmt, cfg.rule))
            del w
        layers.append(make_layer(cfg, qs[0], qs[1], pkg))
        if cfg.w_fmt == "fp8_block" and args.weight_layout == "tiled":
            # its GEMMs read the tiled copies (the MXFP4 layers decode on GEMVs over rows)
            lay = layers[-1]
            lay.w13_tiled, lay.w13_scale_tiled = pkg.tile_weights(lay.w13, None, cfg.w_fmt)
            lay.w2_tiled, lay.w2_scale_tiled = pkg.tile_weights(lay.w2, None, cfg.w_fmt)
        x = synth.activations(cfg)
        i, wt = synth.routing(cfg)
        xs.append(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda())
        ids_l.append(torch.from_numpy(i).cuda())
        ws_l.append(torch.from_numpy(wt).cuda())
        t = len(np.unique(i))
        touched.append(t)
        b13, b2 = expert_bytes(cfg)
        wbytes += t * (b13 + b2)
    torch.cuda.synchronize()
    log(f"built {len(cfgs)} layers in {time.perf_counter() - t0:.1f} s, "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB resident")
    st = LayerStack(layers, xs, ids_l, ws_l)
    T = cfgs[0].tokens
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        st.eager()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.stack_steps):
        st.eager()
    stop.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / args.stack_steps
    st.capture()
    for _ in range(2):
        st.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.stack_steps):
        st.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.stack_steps
    # per-stage times of one layer of each format (the library's stage events)
    timer = pkg.StageTimer()
    per_fmt = {}
    for fmt in ("mxfp4", "fp8_block"):
        l = next(j for j, c in enumerate(cfgs) if c.w_fmt == fmt) if any(c.w_fmt == fmt for c in cfgs) else None
        if l is None:
            continue
        acc = {k: 0.0 for k in pkg.STAGES}
        for _ in range(5):
            pkg.moe_forward_profiled(layers[l], xs[l], ids_l[l], ws_l[l], st.workspace, st.ys[l], timer)
            torch.cuda.synchronize()
            for k, v in timer.durations().items():
                acc[k] += v / 5
        b13, b2 = expert_bytes(cfgs[l])
        per_fmt[fmt] = {"layer": l, "stages_ms": acc, "touched_experts": touched[l],
                        "gate_up_GBps": touched[l] * b13 / (acc["gate_up"] * 1e-3) / 1e9}
    mx = per_fmt.get("mxfp4")
    roof = None
    if mx:
        b13 = expert_bytes(cfgs[mx["layer"]])[0]
        ach = mx["gate_up_GBps"]
        roof = {"bound": "hbm", "kernel": "gemv_gateup_kernel<MXFP4> on the dequantized MXFP8 x (36 of the 48 layers)",
                "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": None, "bytes_per_launch": mx["touched_experts"] * b13,
                "unit_of_work": f"{mx['touched_experts']} touched experts x {b13} B of MXFP4 gate_up weights"}
    n_fp8 = sum(c.w_fmt == "fp8_block" for c in cfgs)
    out = {"workload": f"decode through a {len(cfgs)}-layer routed-expert stack: {len(cfgs) - n_fp8} MXFP4 x "
                       f"MXFP8 layers and {n_fp8} block-FP8 x FP8 layers ({list(synth.FP8_ROUTED_LAYERS)}), "
                       f"512 experts, top-10, hidden 2560, inter 640, {T} tokens, one HIP graph per step",
           "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "steps": args.stack_steps,
           "eager_ms_per_step": eager_ms, "dtype": "fp8",
           "roofline": roof,
           "step_hbm": {"weight_bytes": wbytes, "GBps": wbytes / (ms * 1e-3) / 1e9,
                        "frac": wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "touched_experts_mean": float(np.mean(touched))},
           "per_format_layer": per_fmt}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the stack (first token, first layers)")
        from oracle import moe
        t0 = time.perf_counter()
        done = 0
        for cfg in cfgs:
            i, wt = synth.routing(cfg)
            touched1 = sorted({int(e) for e in i[0]})
            w13, w2 = synth.layer_weights(cfg, experts=touched1)
            pos = {e: j for j, e in enumerate(touched1)}
            x = synth.activations(cfg)[:1]
            ol = dict(w_fmt=cfg.w_fmt, a_fmt=cfg.a_fmt, num_experts=cfg.num_experts, hidden=cfg.hidden,
                      inter=cfg.inter,
                      w13=lambda e, w=w13, c=cfg, p=pos: moe.quantize_expert_weight(w[p[e]], c.w_fmt, c.rule),
                      w2=lambda e, w=w2, c=cfg, p=pos: moe.quantize_expert_weight(w[p[e]], c.w_fmt, c.rule))
            moe.moe_forward(ol, x, i[:1], wt[:1])
            done += 1
            if time.perf_counter() - t0 >= args.cpu_budget / 2:
                break
        el = time.perf_counter() - t0
        per_layer = el / done
        out["cpu_baseline"] = {"value": 1.0 / (per_layer * len(cfgs)), "unit": "tokens/s",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"1 token through the first {done} layer(s) ({el:.1f} s, weights of the "
                                         f"token's experts drawn on the host and quantized by the oracle inside "
                                         f"the timing), scaled to {len(cfgs)} layers"}
    del st, layers
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill_nvfp4", "prefill_mxfp4", "prefill_fp8", "stream_quant",
                             "sweep_quant", "stack_decode", "copy"],
                    help="'all': the decode headline plus every other workload under 'workloads'; "
                         "'copy': a plain 1 GiB device copy that calibrates the HBM byte counters")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-copies", type=int, default=2)
    ap.add_argument("--weight-layout", choices=["tiled", "rows"], default="tiled",
                    help="prefill and the stack's block-FP8 layers: expert weights in the tiled order of "
                         "moe_fp4_tile_weights "
                         "(made once per layer) or row-major")
    ap.add_argument("--stream-layers", type=int, default=48)
    ap.add_argument("--stack-layers", type=int, default=48)
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--sweep-layers", type=int, default=16,
                    help="layers of the streaming workload under the scale-sweep rule")
    ap.add_argument("--copies", type=int, default=8,
                    help="resident copies of the quantized layer rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true",
                    help="streaming workloads: skip the error statistics (for counter runs that must see "
                         "only the timed kernels)")
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
    if args.workload == "copy":
        print(json.dumps(bench_copy(args, torch)), flush=True)
        return
    if args.workload in ("all", "decode"):
        dargs = argparse.Namespace(**vars(args))
        dargs.workload = "decode"
        out = bench_decode(dargs, torch, pkg)
        torch.cuda.empty_cache()
        others = (["prefill_nvfp4", "prefill_mxfp4", "prefill_fp8", "stream_quant", "sweep_quant", "stack_decode"]
                  if args.workload == "all" else [])
    else:
        out = None
        others = [args.workload]
    extra = {}
    for name in others:
        log(f"workload {name}")
        if name == "stream_quant":
            extra[name] = bench_stream_quant(args, torch, pkg)
        elif name == "sweep_quant":
            extra[name] = bench_stream_quant(args, torch, pkg, rule="sweep")
        elif name == "stack_decode":
            extra[name] = bench_stack(args, torch, pkg)
        else:
            extra[name] = bench_prefill(name, args, torch, pkg)
        torch.cuda.empty_cache()
    if out is None:
        name = others[0]
        w = extra[name]
        out = {"metric": METRIC, "value": w["value"], "unit": w["unit"], "n_gpus": 1,
               "steps": w.get("steps", w.get("layers")), "warmup": 2,
               "ms_per_step": w.get("ms_per_step", w.get("ms_per_layer")), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": w.get("dtype", "bf16"), "data": "synthetic",
               "config": {"workload": w["workload"]}, "roofline": w["roofline"]}
        if "cpu_baseline" in w:
            out["cpu_baseline"] = w["cpu_baseline"]
        out["workloads"] = {name: w}
    else:
        out["workloads"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
