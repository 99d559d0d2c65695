"""Write expected outputs of the 8192-token NVFP4 W4A4 layer (512 experts,
top-5, biased router, MXFP8 shared expert) for sampled tokens, computed by the
oracle only.  The NVFP4 tensor scale of h is taken over all 40,960 (token,
expert) rows, so every row's h is computed; the down projection and combine
run for the sampled tokens.

Usage: python tests/golden/make_prefill_golden.py   (about 5-10 min on 8 cores)
Writes tests/golden/prefill_nvfp4_sampled.npz.
"""
import concurrent.futures as cf
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import moe  # noqa: E402

SAMPLE = [0, 1, 1234, 4096, 8191]
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "prefill_nvfp4_sampled.npz")


def _quant_expert(args):
    cfg, e = args
    w13, w2 = synth.expert_weights(cfg, e)
    return e, moe.quantize_expert_weight(w13, cfg.w_fmt, cfg.rule), moe.quantize_expert_weight(w2, cfg.w_fmt, cfg.rule)


def main():
    cfg = synth.CONFIGS["prefill_nvfp4"]
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    touched = sorted(set(int(e) for e in np.unique(ids)))
    t0 = time.time()
    q13, q2 = {}, {}
    with cf.ProcessPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        for e, a, b in ex.map(_quant_expert, [(cfg, e) for e in touched], chunksize=4):
            q13[e], q2[e] = a, b
    print(f"quantized {len(touched)} experts in {time.time() - t0:.0f} s", flush=True)
    s13, s2, gate = synth.shared_expert(cfg)
    shared = dict(w13=moe.quantize_expert_weight(s13, "mxfp8"), w2=moe.quantize_expert_weight(s2, "mxfp8"),
                  gate_bits=gate)
    layer = dict(w_fmt=cfg.w_fmt, a_fmt=cfg.a_fmt, num_experts=cfg.num_experts, hidden=cfg.hidden,
                 inter=cfg.inter, w13=lambda e: q13[e], w2=lambda e: q2[e], shared=shared)
    t0 = time.time()
    y, st = moe.moe_forward(layer, x, ids, wts, sample_tokens=SAMPLE, return_stages=True)
    print(f"forward in {time.time() - t0:.0f} s", flush=True)
    np.savez_compressed(OUT, sample=np.array(SAMPLE), y=y, s_x=np.float32(st["xrec"]["tensor_scale"]),
                        s_h=np.float32(st["hrec"]["tensor_scale"]),
                        counts=np.diff(st["offsets"]).astype(np.int32))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
