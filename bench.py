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


class StepEvents:
    """n HIP events recorded on the current stream between steps, created
    without the system-scope fence (a default event's release writes back the
    L2 at every record, several microseconds on a decode step), for per-step
    times: median and p10 / p90."""

    def __init__(self, n):
        import ctypes

        from block_scaled_fp4_nvfp4_amd import _lib
        self._ct = ctypes
        self._hip = _lib._hip_runtime()
        if self._hip is None:
            raise RuntimeError("HIP runtime library not found")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(e), _lib._HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e.value)

    def record(self, i, torch):
        st = self._ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        if self._hip.hipEventRecord(self._ct.c_void_p(self.ev[i]), st) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i, j):
        out = self._ct.c_float()
        if self._hip.hipEventElapsedTime(self._ct.byref(out), self._ct.c_void_p(self.ev[i]),
                                         self._ct.c_void_p(self.ev[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def __del__(self):
        for e in getattr(self, "ev", []):
            self._hip.hipEventDestroy(self._ct.c_void_p(e))


def step_distribution(torch, step, steps):
    """Times each of `steps` calls of step(i) between events; returns the
    median, p10 and p90 in ms (event records add well under a microsecond)."""
    import numpy as np
    ev = StepEvents(steps + 1)
    torch.cuda.synchronize()
    ev.record(0, torch)
    for i in range(steps):
        step(i)
        ev.record(i + 1, torch)
    torch.cuda.synchronize()
    t = np.array([ev.ms(i, i + 1) for i in range(steps)])
    return {"median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)), "steps": steps}


def timed_oracle(fn, budget_s):
    """fn() repeated for about budget_s seconds, once with the BLAS thread
    pool at its default size (all host cores) and once limited to one
    thread; returns (all-cores (reps, seconds), one-core (reps, seconds),
    threads of the first)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    out = []
    for limit in (None, 1):
        with threadpool_limits(limits=limit):
            t0 = time.perf_counter()
            reps = 0
            while True:
                fn()
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget_s or reps >= 50:
                    break
        out.append((reps, el))
    return out[0], out[1], threads


def _oracle_quantize_task(task):
    """Worker of the streaming workload's oracle leg: the oracle's NVFP4
    quantization of one expert's gate_up and down bf16 tensors."""
    w13_bits, w2_bits, rule = task
    sys.path.insert(0, ROOT)
    from oracle import quant
    from oracle.formats import bf16_to_f64, pack_nibbles
    out = []
    for w in (w13_bits, w2_bits):
        q = quant.quantize_nvfp4(bf16_to_f64(w), rule)
        out.append((pack_nibbles(q["codes"]), q["scales"], float(q["tensor_scale"]),
                    quant.dequantize_nvfp4(q["codes"], q["scales"], q["tensor_scale"])))
    return out


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
    (reps, el), (reps1, el1), threads = timed_oracle(lambda: moe.moe_forward(layer, x_s, ids_s, wts_s),
                                                     budget_s / 2)
    sample = (f"{n} token(s) of the {cfg.name} layer forward (dequantize-then-matmul in float64, weights "
              f"pre-quantized by the oracle)")
    return {"value": reps * n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cores": cores, "sample": f"{sample}: {reps} repeat(s), {el:.1f} s",
            "single_core": {"value": reps1 * n / el1, "unit": "tokens/s", "cores": 1, "blas_threads": 1,
                            "sample": f"{sample}: {reps1} repeat(s), {el1:.1f} s"}}


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
    eager_ms = start.elapsed_time(stop) / args.steps
    # the timed steps: the same K forwards (layer copies in turn) captured as
    # one HIP graph and replayed, as a serving runtime runs decode (the
    # MXFP4-FP8-R12 card's deployment table: decode CUDA graphs); eager
    # launches leave the GPU idle for a few microseconds at each call
    from block_scaled_fp4_nvfp4_amd.stack import LayerStack
    n = args.steps
    gstack = LayerStack([layers[i % len(layers)] for i in range(n)], [x] * n, [tid] * n, [tw] * n)
    gstack.capture()
    gstack.replay()
    torch.cuda.synchronize()
    start.record()
    gstack.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    del gstack

    # per-stage durations (events recorded by the library between its launches)
    timer = pkg.StageTimer()
    acc = {s: 0.0 for s in pkg.STAGES}
    for i in range(args.steps):
        pkg.moe_forward_profiled(layers[i % len(layers)], x, tid, tw, ws, y, timer)
        torch.cuda.synchronize()
        for k, v in timer.durations().items():
            acc[k] += v
    stages = {k: v / args.steps for k, v in acc.items()}
    dist = step_distribution(torch, lambda i: pkg.moe_forward(layers[i % len(layers)], x, tid, tw, ws, y),
                             args.steps)

    touched = len(np.unique(ids))
    b13, b2 = expert_bytes(cfg)
    P = T * cfg.top_k
    gateup_bytes = touched * b13 + T * cfg.hidden * 2 + P * cfg.inter * 4
    down_bytes = touched * b2 + P * cfg.inter * 4 + P * cfg.hidden * 4
    step_bytes = touched * (b13 + b2) + T * cfg.hidden * 2 + T * cfg.hidden * 4
    gu_ms = stages["gate_up"]
    tr = measured_traffic("gemv_gateup_kernel", "gate_up", "decode")
    roof = {"bound": "hbm", "kernel": "gemv_gateup_kernel<NVFP4, 5>", "scope": "the gate_up GEMV kernel alone",
            "achieved": gateup_bytes / (gu_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": tr["bytes_per_launch"] if tr else None,
            "bytes_per_launch": gateup_bytes,
            "unit_of_work": f"{touched} touched experts x {b13} B of NVFP4 gate_up weights"
                            f" + x {T * cfg.hidden * 2} B + h {P * cfg.inter * 4} B"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the whole layer step (every kernel of moe_fp4_forward) against the same peak
    roof["layer"] = {"bytes": step_bytes, "achieved": step_bytes / (ms * 1e-3) / 1e9,
                     "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "unit_of_work": f"{touched} touched experts x {b13 + b2} B + x + y"}
    out = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.num_experts} experts, top-{cfg.top_k}, hidden "
                               f"{cfg.hidden}, inter {cfg.inter}, {T} tokens, {cfg.w_fmt} "
                               f"({cfg.rule}) weights x bf16 activations",
                   "tokens": T, "touched_experts": int(touched), "layer_copies": len(layers),
                   "timing": "the K steps captured as one HIP graph: one untimed replay, then the timed one"},
        "eager_ms_per_step": eager_ms,
        "roofline": roof,
        "step_hbm": {"bytes": step_bytes, "GBps": step_bytes / (ms * 1e-3) / 1e9,
                     "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "stages_ms": stages,
        "step_distribution": dist,
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
    dist = step_distribution(torch, lambda i: pkg.moe_forward(layers[i % len(layers)], x, tid, tw, ws, y), steps)
    timer = pkg.StageTimer()
    acc = {s_: 0.0 for s_ in pkg.STAGES}
    for i in range(steps):
        pkg.moe_forward_profiled(layers[i % len(layers)], x, tid, tw, ws, y, timer)
        torch.cuda.synchronize()
        for k_, v in timer.durations().items():
            acc[k_] += v
    return ms, {k_: v / steps for k_, v in acc.items()}, dist


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
    ms, stages, dist = time_steps(pkg, torch, layers, x, tid, tw, ws, y, args.prefill_steps, 2)
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
    # the gate_up kernel as the kernel trace names it (last parameter: output
    # tiles per workgroup, 1 for gate_up)
    gk = {"nvfp4": "grouped_gemm_nv2_kernel<0, 2, 20, WT, 1>", "mxfp4": "grouped_gemm_mx2_kernel<1, 0, 2, 20, WT, 1>",
          "fp8_block": "grouped_gemm_mx2_kernel<2, 0, 2, 20, WT, 1>"}[cfg.w_fmt].replace("WT", str(tiled).lower())
    roof = {"bound": "mfma", "kernel": gk + " (gate_up)", "mfma_dtype":
            {"bf16": "fp16 (exact NVFP4 decode)", "fp8": "fp8 x fp4" if cfg.w_fmt == "mxfp4" else "fp8"}[peak_key],
            "achieved": flops_gu / (gu_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
            "traffic": (lambda t: t["bytes_per_launch"] if t else None)(
                measured_traffic(gk.split("<")[0], "gate_up", name)),
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
           "roofline": roof, "stages_ms": stages, "step_distribution": dist,
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


def measured_traffic(kernel, stage, workload):
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
        if kv.get("kernel") != kernel or kv.get("stage") != stage or kv.get("workload") != workload:
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


def bench_ceilings(args, torch, pkg):
    """Measured device ceilings (include/fp4moe_probe.h): a streaming read
    over 4 GiB (larger than the 256 MB Infinity Cache) at several grid sizes,
    the issue rate of each MFMA operand type the kernels use, and the
    routing-weighted combine as a store of o plus a combine pass against fp32
    atomics into y, at the prefill and decode shapes."""
    import ctypes

    import numpy as np
    L = pkg.lib()
    vp = ctypes.c_void_p
    L.fp4_probe_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
    L.fp4_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    L.fp4_probe_combine.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    stream = lambda: vp(torch.cuda.current_stream().cuda_stream)

    def timeit(fn, reps=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def ok(st):
        if st != 0:
            raise RuntimeError(L.fp4_last_error().decode())

    out = {"metric": "measured device ceilings", "unit": "GB/s and TFLOP/s"}
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    reads = {}
    for grid in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        ms = timeit(lambda: ok(L.fp4_probe_read(vp(buf.data_ptr()), nbytes, grid, vp(sink.data_ptr()), stream())))
        reads[grid] = nbytes / (ms * 1e-3) / 1e9
    out["stream_read_GBps"] = {"by_grid": reads, "best": max(reads.values()), "bytes": nbytes,
                               "peak_spec": HBM_PEAK_GBS, "frac_of_spec": max(reads.values()) / HBM_PEAK_GBS}
    del buf
    grid, iters = 2048, 2000
    acc = torch.empty(grid * 256 * 4, dtype=torch.float32, device="cuda")
    clk = torch.zeros(128, dtype=torch.int64, device="cuda")
    kinds = {"f16": (0, 16384, 2500.0), "bf16": (1, 16384, 2500.0), "fp8_x_fp8": (2, 65536, 5000.0),
             "fp8_x_fp4": (3, 65536, 5000.0), "fp4_x_fp4": (4, 65536, 10100.0),
             "f16_32x32x16": (5, 32768, 2500.0), "fp8_x_fp8_32x32x64": (6, 131072, 5000.0),
             "fp4_x_fp4_32x32x64": (7, 131072, 10100.0)}
    mf = {}
    for name, (kind, flops, peak) in kinds.items():
        ms = timeit(lambda: ok(L.fp4_probe_mfma(kind, iters, grid, vp(acc.data_ptr()), vp(clk.data_ptr()),
                                                stream())), reps=5)
        tf = grid * 4 * iters * 8 * flops / (ms * 1e-3) / 1e12
        c = clk.cpu().numpy().reshape(64, 2).astype(np.float64)
        ghz = 0.1 * c[:, 0].sum() / c[:, 1].sum()  # shader cycles per 100 MHz tick, last launch
        # cycles one SIMD spends per instruction at that clock (256 CUs x 4 SIMDs)
        cyc = flops * 1024 * ghz * 1e9 / (tf * 1e12)
        mf[name] = {"TFLOPs": tf, "peak_spec": peak, "frac_of_spec": tf / peak, "clock_GHz": ghz,
                    "simd_cycles_per_instruction": cyc}
    out["mfma_TFLOPs"] = mf
    rng = np.random.default_rng(1)
    comb = {}
    for T, k in ((8192, 10), (8192, 5), (16, 10)):
        E, H = 512, 2560
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        por = np.argsort(ids.reshape(-1), kind="stable").astype(np.int32)
        rop = np.empty_like(por)
        rop[por] = np.arange(T * k, dtype=np.int32)
        w = np.full(T * k, 0.1, np.float32)
        d_por, d_rop, d_w = (torch.from_numpy(a).cuda() for a in (por, rop, w))
        o = torch.empty(T * k, H, dtype=torch.float32, device="cuda")
        y = torch.zeros(T, H, dtype=torch.float32, device="cuda")
        args_ = lambda mode: (mode, vp(d_por.data_ptr()), vp(d_rop.data_ptr()), vp(d_w.data_ptr()), T, k, H,
                              vp(o.data_ptr()), vp(y.data_ptr()), stream())
        t_store = timeit(lambda: ok(L.fp4_probe_combine(*args_(0))))
        t_comb = timeit(lambda: ok(L.fp4_probe_combine(*args_(1))))
        t_zero = timeit(lambda: y.zero_())
        t_atom = timeit(lambda: ok(L.fp4_probe_combine(*args_(2))))
        y.zero_()
        ok(L.fp4_probe_combine(*args_(2)))
        ya = y.clone()
        ok(L.fp4_probe_combine(*args_(0)))
        ok(L.fp4_probe_combine(*args_(1)))
        torch.cuda.synchronize()
        comb[f"T{T}_k{k}"] = {"store_o_us": t_store * 1e3, "combine_us": t_comb * 1e3,
                              "store_plus_combine_us": (t_store + t_comb) * 1e3,
                              "zero_y_us": t_zero * 1e3, "atomic_into_y_us": t_atom * 1e3,
                              "max_abs_diff": float((ya - y).abs().max())}
    out["combine_experiment"] = comb
    return out


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
        if layer == 0 and not args.no_cpu_baseline:
            # the oracle leg below quantizes these very tensors (the first
            # experts of layer 0) and compares with the GPU's bytes
            ne = args.oracle_experts
            kept = {"w13": w13[:ne].view(torch.int16).cpu().numpy().view(np.uint16),
                    "w2": w2[:ne].view(torch.int16).cpu().numpy().view(np.uint16)}
            for nm, q, w in (("q13", q13, w13), ("q2", q2, w2)):
                sub = {k: q[k][:ne] for k in ("codes", "scales", "tensor_scale")}
                be = pkg.block_error(w[:ne], sub, "nvfp4").double().sum(dim=(1, 2))
                kept[nm] = {k: v.cpu().numpy() for k, v in sub.items()}
                kept[nm]["sq_err"] = be.cpu().numpy()
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
                            measured_traffic("quant_fp4_kernel", "quantize", "stream_quant" if rule == "4over6" else "sweep_quant")),
                        "bytes_per_layer": bytes_layer,
                        "unit_of_work": "2 B read + 0.5625 B written per value (+4 B per tensor)"},
           "quality": {"per_tensor_rel_err": {n: {"mean": m, "max": mx} for n, m, mx, *_ in stats},
                       "m4_fraction": float(np.mean([st[3] for st in stats])) if stats else None}}
    if rule != "4over6" and stats:
        out["quality"]["per_tensor_rel_err_4over6_same_data"] = {st[0]: {"mean": st[6]} for st in stats}
        out["quality"]["note"] = ("m4_fraction: blocks whose scale is not the amax/6 plan's; "
                                  "first and last layer")
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on streaming quantization ({rule}) and checking the GPU's bytes")
        import multiprocessing as mp
        ne = kept["w13"].shape[0]
        tasks = [(kept["w13"][e], kept["w2"][e], rule) for e in range(ne)]
        cores = len(os.sched_getaffinity(0))
        procs = max(1, min(16, cores, ne))
        t0 = time.perf_counter()
        with mp.get_context("spawn").Pool(procs) as pool:
            res = pool.map(_oracle_quantize_task, tasks)
        el = time.perf_counter() - t0
        n1 = max(1, min(ne, 2))
        t1 = time.perf_counter()
        for t in tasks[:n1]:
            _oracle_quantize_task(t)
        el1 = time.perf_counter() - t1
        vals_e = 3 * H * I
        ok_codes = ok_scales = ok_ts = True
        rel_gpu, rel_orc = [], []
        for e in range(ne):
            for j, (nm, wk) in enumerate((("q13", "w13"), ("q2", "w2"))):
                codes, scales, ts, deq = res[e][j]
                g = kept[nm]
                ok_codes &= bool(np.array_equal(codes, g["codes"][e]))
                ok_scales &= bool(np.array_equal(scales, g["scales"][e]))
                ok_ts &= bool(np.float32(ts) == g["tensor_scale"][e])
                src = (kept[wk][e].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                nrm = float((src * src).sum())
                rel_orc.append(float(np.sqrt(((src - deq) ** 2).sum() / nrm)))
                rel_gpu.append(float(np.sqrt(g["sq_err"][e] / nrm)))
        out["oracle_check"] = {
            "tensors": f"gate_up and down of experts 0..{ne - 1} of layer 0, copied back from the device "
                       f"after the timed quantization",
            "codes_equal": ok_codes, "scales_equal": ok_scales, "tensor_scales_equal": ok_ts,
            "rel_err_gpu_mean": float(np.mean(rel_gpu)), "rel_err_oracle_mean": float(np.mean(rel_orc)),
            "rel_err_max_abs_diff": float(np.max(np.abs(np.array(rel_gpu) - np.array(rel_orc))))}
        out["cpu_baseline"] = {"value": ne * vals_e * 2.5625 / el / 1e9, "unit": "GB/s",
                               "values_per_s": ne * vals_e / el, "cores": procs, "kind": "oracle",
                               "sample": f"{ne} experts of layer 0 (the device tensors above, gate_up + down), "
                                         f"one expert per process of a {procs}-process pool, {el:.1f} s "
                                         f"(process start included)",
                               "single_core": {"value": n1 * vals_e * 2.5625 / el1 / 1e9, "unit": "GB/s",
                                               "cores": 1, "sample": f"{n1} of those experts in this process, "
                                                                     f"{el1:.1f} s"}}
    return out


def bench_hessian_quant(args, torch, pkg):
    """One layer of 512 experts (fused gate_up 1280 x 2560, down 2560 x 640;
    bf16 Student-t(4) source with 1% outlier rows x8, as the streaming
    workload) quantized to NVFP4 by the Hessian-weighted scale search, with
    synthetic calibration covariances drawn on the device per expert (the
    recipe of synth.calibration_hessian, estimated from 256 sampled rows)
    and calibration row counts from synth.calibration_rows (two thin
    experts keep plain max)."""
    import numpy as np

    import synth
    E, H, I = 512, 2560, 640
    gen = torch.Generator(device="cuda")
    tdist = torch.distributions.StudentT(torch.tensor(4.0, device="cuda"))

    def source(rows, cols, seed):
        gen.manual_seed(seed)
        torch.manual_seed(seed + 1)
        v = tdist.sample((E, rows, cols)) * (0.02 / 2 ** 0.5)
        n_out = int(round(0.01 * rows))
        idx = torch.argsort(torch.rand(E, rows, device="cuda", generator=gen), dim=1)[:, :n_out]
        v.scatter_(1, idx[:, :, None].expand(E, n_out, cols), v.gather(1, idx[:, :, None].expand(E, n_out, cols)) * 8)
        return v.to(torch.bfloat16)

    def hessians(cols, n_rows, seed, sample=256):
        nb = cols // 16
        out = torch.empty(E, nb, 16, 16, dtype=torch.float32, device="cuda")
        gen.manual_seed(seed)
        for e0 in range(0, E, 32):
            ne = min(32, E - e0)
            scale = torch.exp(0.5 * torch.randn(ne, 1, cols, device="cuda", generator=gen))
            c = torch.rand(ne, 1, nb, device="cuda", generator=gen)
            z = torch.randn(ne, sample, cols, device="cuda", generator=gen)
            sh = torch.randn(ne, sample, nb, device="cuda", generator=gen)
            a = ((z + (c * sh).repeat_interleave(16, dim=2)) * scale).to(torch.bfloat16).double()
            a = a.view(ne, sample, nb, 16)
            out[e0:e0 + ne] = (torch.einsum("etbi,etbj->ebij", a, a) / sample).float()
        out[torch.from_numpy(n_rows == 0).cuda()] = 0.0
        return out

    n_rows = synth.calibration_rows(11, E)
    rows_dev = torch.from_numpy(n_rows).cuda()
    w13, w2 = source(2 * I, H, 3000), source(H, I, 3100)
    h13, h2 = hessians(H, n_rows, 3200), hessians(I, n_rows, 3300)
    torch.cuda.synchronize()
    for _ in range(1):
        pkg.quantize_hessian(w13, h13, rows_dev)
        pkg.quantize_hessian(w2, h2, rows_dev)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = args.hessian_reps
    start.record()
    for _ in range(reps):
        q13 = pkg.quantize_hessian(w13, h13, rows_dev, want_choice=True)
        q2 = pkg.quantize_hessian(w2, h2, rows_dev, want_choice=True)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    vals = E * 3 * H * I
    hbytes = h13.numel() * 4 + h2.numel() * 4
    alg_bytes = vals * 2.5625 + hbytes + E * 8 + E * 4 * 2
    gbs = alg_bytes / (ms * 1e-3) / 1e9

    # fp64 FMAs the search spends: 152 per candidate (136 for t = T d over the
    # upper triangle T of H + H^T, 16 for d . t) of every block whose
    # window holds more than one code (the amax/6 and block-max-to-4 plans'
    # codes, from the block maxima and the tensor scales; thin experts none)
    def fmas(w, q, full):
        amax_b = w.float().abs().view(E, -1, 16).amax(dim=2)
        S = q["tensor_scale"].view(E, 1)
        c6 = torch.clamp(amax_b / (6 * S), max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).int()
        c4 = torch.clamp(amax_b / (4 * S), max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).int()
        width = torch.where(full.view(E, 1), c4 - c6 + 1, torch.ones_like(c4))
        return float(torch.where(width > 1, width, torch.zeros_like(width)).sum()) * 152

    full = torch.from_numpy(n_rows >= 64).cuda()
    n_fma = fmas(w13, q13, full) + fmas(w2, q2, full)
    tflops = 2 * n_fma / (ms * 1e-3) / 1e12
    # quality on the first experts: relative plain and H-weighted error of the
    # Hessian search, the plain sweep, 4/6 and plain max on the same tensors
    qual = {}
    ne = 8
    for name, w, hh in () if args.no_quality else (("gate_up", w13[:ne].contiguous(), h13[:ne]),
                                                    ("down", w2[:ne].contiguous(), h2[:ne])):
        x = w.double()
        xv = x.view(ne, x.shape[1], -1, 16)
        hx = torch.einsum("erbi,ebij,erbj->e", xv, hh.double(), xv)
        res = {}
        cand = {"hessian": pkg.quantize_hessian(w, hh, rows_dev[:ne])}
        for rule in ("sweep", "4over6", "rtn"):
            cand[rule] = pkg.quantize(w, "nvfp4", rule)
        for rule, q in cand.items():
            d = (x - pkg.dequantize(q, "nvfp4", tuple(w.shape)).double()).view(ne, x.shape[1], -1, 16)
            hd = torch.einsum("erbi,ebij,erbj->e", d, hh.double(), d)
            full_e = full[:ne]
            res[rule] = {"rel_err": float((d.pow(2).sum(dim=(1, 2, 3)) / x.pow(2).sum(dim=(1, 2))).sqrt()[full_e].mean()),
                         "rel_weighted_err": float((hd / hx).sqrt()[full_e].mean())}
        qual[name] = res
    out = {"workload": f"Hessian-weighted NVFP4 quantization of one layer: {E} experts x (gate_up {2 * I}x{H}, "
                       f"down {H}x{I}), bf16 Student-t(4) source with 1% outlier rows x8, synthetic per-expert "
                       f"calibration covariances (16x16 diagonal blocks of the input Hessian)",
           "value": gbs, "unit": "GB/s", "ms_per_layer": ms, "reps": reps, "dtype": "f64",
           "roofline": {"bound": "alu", "kernel": "hessian_quant_kernel",
                        "achieved": tflops, "peak": 78.6, "unit": "TFLOP/s", "frac": tflops / 78.6,
                        "traffic": (lambda t: t["bytes_per_launch"] if t else None)(
                            measured_traffic("hessian_quant_kernel", "quantize", "hessian_quant")),
                        "traffic_unit": "HBM bytes per layer", "flops_per_layer": 2 * n_fma,
                        "unit_of_work": "2 x 152 fp64 FLOPs per candidate scale of each block whose "
                                        "window holds more than one code"},
           "bytes_per_layer": alg_bytes,
           "thin_experts": int((n_rows < 64).sum()),
           "quality_first_experts": qual}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the Hessian-weighted search")
        from oracle import quant
        from oracle.formats import bf16_to_f64
        t0 = time.perf_counter()
        n_vals = 0
        e = 0
        while time.perf_counter() - t0 < args.cpu_budget and e < 8:
            w13h, w2h = synth.streaming_expert(0, e)
            for w, cols in ((w2h, I), (w13h, H)):
                hh = synth.calibration_hessian(11, e, cols, 256)
                quant.quantize_nvfp4_hessian(bf16_to_f64(w), hh, 256)
                n_vals += w.size
                if time.perf_counter() - t0 >= args.cpu_budget:
                    break
            e += 1
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n_vals * 2.5625 / el / 1e9, "unit": "GB/s", "values_per_s": n_vals / el,
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"{n_vals} values of layer-0 experts (down then gate_up), source and "
                                         f"covariances drawn on the host, {el:.1f} s"}
    del w13, w2, h13, h2
    torch.cuda.empty_cache()
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


def pmc_summary(dirs, num_xcd=8, num_cu=256, simd_per_cu=4):
    """Per-kernel table from rocprofv3 --pmc counter CSVs (a directory per
    pass; averages over a kernel's dispatches).  The normalisations are those
    of rocprofv3's own derived metrics: the CSV's GRBM_GUI_ACTIVE is summed over
    the XCDs, so per XCD it is / num_xcd; MFMA busy = sum of
    SQ_VALU_MFMA_BUSY_CYCLES / (GUI x SIMDs) (MfmaUtil); VALU busy = sum of
    SQ_ACTIVE_INST_VALU / (GUI x CUs) (VALUBusy); LDS bank conflicts per access
    = conflict / (active - conflict) cycles (LdsBankConflict); L2 hit = hits /
    (hits + misses); waits are fractions of SQ_WAVE_CYCLES.  MFMA FLOPs per
    operand type = SQ_INSTS_VALU_MFMA_MOPS_<type> x 512."""
    import csv
    import glob
    from collections import defaultdict
    per = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
            with open(path) as f:
                for r in csv.DictReader(f):
                    k = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("fp4::", "")
                    per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    rows = []
    for k, cs in per.items():
        a = {c: sum(v) / len(v) for c, v in cs.items()}
        if "SQ_INSTS_MFMA" in a and a["SQ_INSTS_MFMA"] == 0:
            continue
        gui = a.get("GRBM_GUI_ACTIVE", 0.0) / num_xcd
        row = {"kernel": k, "dispatches": min(len(v) for v in cs.values()), "gui_cycles": gui}
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in a:
            row["mfma_busy"] = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * num_cu * simd_per_cu)
        if gui and "SQ_ACTIVE_INST_VALU" in a:
            row["valu_busy"] = a["SQ_ACTIVE_INST_VALU"] / (gui * num_cu)
        if gui and "SQ_BUSY_CU_CYCLES" in a:
            row["cu_busy"] = a["SQ_BUSY_CU_CYCLES"] / (gui * num_cu)
        if "SQ_WAVE_CYCLES" in a:
            for c, n in (("SQ_WAIT_INST_ANY", "wait_any"), ("SQ_WAIT_INST_LDS", "wait_lds")):
                if c in a:
                    row[n] = a[c] / a["SQ_WAVE_CYCLES"]
        if "SQ_LDS_BANK_CONFLICT" in a and "SQ_LDS_IDX_ACTIVE" in a:
            row["lds_conflicts_per_access"] = a["SQ_LDS_BANK_CONFLICT"] / max(
                a["SQ_LDS_IDX_ACTIVE"] - a["SQ_LDS_BANK_CONFLICT"], 1.0)
        if "TCC_HIT_sum" in a and "TCC_MISS_sum" in a:
            row["l2_hit"] = a["TCC_HIT_sum"] / max(a["TCC_HIT_sum"] + a["TCC_MISS_sum"], 1.0)
        for t in ("F8", "F6F4", "F16", "BF16"):
            c = "SQ_INSTS_VALU_MFMA_MOPS_" + t
            if c in a:
                row["mfma_gflop_" + t.lower()] = a[c] * 512 / 1e9
        if "SQ_INSTS_MFMA" in a:
            row["mfma_insts"] = a["SQ_INSTS_MFMA"]
        if "SQ_INSTS_VALU" in a and a.get("SQ_WAVES"):
            row["valu_insts_per_wave"] = a["SQ_INSTS_VALU"] / a["SQ_WAVES"]
            row["valu_insts"] = a["SQ_INSTS_VALU"]
        rows.append(row)
    return rows


# kernels whose HBM traffic profiles/hbm_traffic.txt records, per workload:
# (kernel, demangled-name prefixes, stage, source file, per): per "launch" is
# the average over the matching dispatches, per "layer" the sum over the run
# divided by the layers run (the quantizer's amax, scale and code kernels)
_QUANT_KERNELS = ("quant_fp4_kernel<", "tensor_amax_kernel<", "amax_parts_kernel<", "nv_scale_from_parts_kernel",
                  "nv_tensor_scale_kernel", "fill_u32_kernel")
TRAFFIC_KERNELS = {
    "decode": [("gemv_gateup_kernel", ("gemv_gateup_kernel<",), "gate_up", "moe.hip", "launch"),
               ("gemv_down_kernel", ("gemv_down_kernel<",), "down", "moe.hip", "launch"),
               ("perm_small_kernel", ("perm_small_kernel",), "permute", "moe.hip", "launch"),
               ("combine_kernel", ("combine_kernel<",), "combine", "moe.hip", "launch")],
    "prefill_nvfp4": [("grouped_gemm_nv2_kernel", ("grouped_gemm_nv2_kernel<0,",), "gate_up", "moe_gemm.hip", "launch"),
                      ("grouped_gemm_nv2_kernel", ("grouped_gemm_nv2_kernel<1,",), "down", "moe_gemm.hip", "launch"),
                      ("combine_f16_kernel", ("combine_f16_kernel<",), "combine", "moe.hip", "launch")],
    "prefill_mxfp4": [("grouped_gemm_mx2_kernel", ("grouped_gemm_mx2_kernel<1, 0,",), "gate_up", "moe_gemm.hip", "launch"),
                      ("grouped_gemm_mx2_kernel", ("grouped_gemm_mx2_kernel<1, 1,",), "down", "moe_gemm.hip", "launch"),
                      ("combine_f16_kernel", ("combine_f16_kernel<",), "combine", "moe.hip", "launch")],
    "prefill_fp8": [("grouped_gemm_mx2_kernel", ("grouped_gemm_mx2_kernel<2, 0,",), "gate_up", "moe_gemm.hip", "launch"),
                    ("grouped_gemm_mx2_kernel", ("grouped_gemm_mx2_kernel<2, 1,",), "down", "moe_gemm.hip", "launch"),
                    ("combine_f16_kernel", ("combine_f16_kernel<",), "combine", "moe.hip", "launch")],
    "stream_quant": [("quant_fp4_kernel", _QUANT_KERNELS, "quantize", "quant.hip", "layer")],
    "sweep_quant": [("quant_fp4_kernel", _QUANT_KERNELS, "quantize", "quant.hip", "layer")],
    "hessian_quant": [("hessian_quant_kernel", ("hessian_quant_kernel<",), "quantize", "hessian.hip", "layer")],
}


def traffic_summary(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, layers=1):
    """hbm_traffic.txt lines from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs
    (one counter per run, KiB per dispatch summed over the XCDs' L2s) of the
    workload and of `bench.py --workload copy` (2^28 float32 read and written
    per launch), which calibrates each counter to bytes."""
    import csv
    import glob

    def per_kernel(d, counter):
        out = {}
        for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        k = r["Kernel_Name"].replace("void ", "").replace("fp4::", "")
                        out.setdefault(k, []).append(float(r["Counter_Value"]))
        return out

    def calib(d, counter):
        vals = [v for k, vs in per_kernel(d, counter).items() if "neg" in k for v in vs]
        return (1 << 30) / (1024.0 * sum(vals) / len(vals))

    fs, ws = calib(copy_fetch_dir, "FETCH_SIZE"), calib(copy_write_dir, "WRITE_SIZE")
    fk, wk = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    lines = []
    for kernel, prefixes, stage, src, per in TRAFFIC_KERNELS[workload]:
        def pick(m):
            v = [x for k, xs in m.items() if k.startswith(prefixes) for x in xs]
            if not v:
                return None
            return (sum(v) / len(v) if per == "launch" else sum(v) / layers) * 1024.0
        f, w = pick(fk), pick(wk)
        if f is None or w is None:
            continue
        rel = "block_scaled_fp4_nvfp4_amd/csrc/" + src
        lines.append(f"kernel={kernel} stage={stage} workload={workload} fetch_bytes={f * fs:.0f} "
                     f"write_bytes={w * ws:.0f} bytes_per_launch={f * fs + w * ws:.0f} copy_scale={fs:.4f} "
                     f"write_scale={ws:.4f} per={per} source={rel} source_sha={file_sha(rel)}")
    return lines


def trace_summary(workload, stats_csv, bench_log, extra=""):
    """profiles/kernels_<workload>.txt from a rocprofv3 --kernel-trace --stats
    run of bench.py: the bench line of the same run and the library's
    kernels by total time (torch's own kernels, which set up the inputs,
    are left out)."""
    import csv
    line = None
    with open(bench_log) as f:
        for ln in f:
            if ln.startswith("{"):
                line = json.loads(ln)
    out = [f"# rocprofv3 kernel trace of the {workload} workload (bench.py defaults for it{extra and ', ' + extra})",
           f"# command: cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o "
           f"{workload} -- python3 /root/repo/bench.py --workload {workload}{extra and ' ' + extra} --no-cpu-baseline",
           f"# table: python3 /root/repo/bench.py --trace-summary {workload} <out>/{workload}_kernel_stats.csv "
           f"<bench stdout>{extra and ' ' + repr(extra)}"]
    if line:
        w = line.get("workloads", {}).get(workload, line)
        r = w.get("roofline", {})
        ms = w.get("ms_per_step", w.get("ms_per_layer"))
        out.append(f"# bench line of the same run (timed under the profiler): value {w.get('value'):.6g} {w.get('unit')}, ms per "
                   f"{'step' if 'ms_per_step' in w else 'layer'} {ms:.6g}, roofline achieved "
                   f"{r.get('achieved', float('nan')):.6g} {r.get('unit')} (frac {r.get('frac', float('nan')):.4f})")
        out.append(f"# stage times from HIP events in that run (ms): "
                   f"{json.dumps({k: round(v, 4) for k, v in (w.get('stages_ms') or {}).items()})}")
    out.append("#")
    out.append(f"{'kernel':64s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_%':>8s}")
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            name = r["Name"].replace("void ", "")
            if not name.startswith("fp4::"):
                continue
            rows.append((name[5:].split("(")[0], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    for k, c, a, lo, hi, pc in sorted(rows, key=lambda x: -x[1] * x[2]):
        out.append(f"{k[:64]:64s} {c:6d} {a:10.2f} {lo:10.2f} {hi:10.2f} {pc:8.2f}")
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-summary":
        a = sys.argv[2:]
        print("\n".join(trace_summary(a[0], a[1], a[2], a[3] if len(a) > 3 else "")))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        for row in pmc_summary(sys.argv[2:]):
            print(json.dumps(row))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-summary":
        a = sys.argv[2:]
        for line in traffic_summary(a[0], a[1], a[2], a[3], a[4], int(a[5]) if len(a) > 5 else 1):
            print(line)
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill_nvfp4", "prefill_mxfp4", "prefill_fp8", "stream_quant",
                             "sweep_quant", "hessian_quant", "stack_decode", "copy", "ceilings"],
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
    ap.add_argument("--oracle-experts", type=int, default=16,
                    help="streaming workloads: experts of layer 0 copied back and checked against the oracle")
    ap.add_argument("--hessian-reps", type=int, default=3,
                    help="timed repetitions of the Hessian-weighted quantization of one layer")
    ap.add_argument("--copies", type=int, default=8,
                    help="resident copies of the quantized layer rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true",
                    help="streaming and Hessian workloads: skip the error statistics (for counter runs that "
                         "must see only the timed kernels)")
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
    if args.workload == "ceilings":
        print(json.dumps(bench_ceilings(args, torch, pkg)), flush=True)
        return
    if args.workload in ("all", "decode"):
        dargs = argparse.Namespace(**vars(args))
        dargs.workload = "decode"
        out = bench_decode(dargs, torch, pkg)
        torch.cuda.empty_cache()
        others = (["prefill_nvfp4", "prefill_mxfp4", "prefill_fp8", "stream_quant", "sweep_quant", "hessian_quant",
                   "stack_decode"]
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
        elif name == "hessian_quant":
            extra[name] = bench_hessian_quant(args, torch, pkg)
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
