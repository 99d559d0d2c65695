"""A forward captured into a HIP graph before any eager call in the process:
the one-time per-device set-up (dynamic-LDS limits of the GEMM kernels, the
shared expert's helper stream and events) then happens inside the capture.
Run in a fresh interpreter so that nothing has been launched before; the
replays must equal an eager forward bit for bit."""
import os
import subprocess
import sys

import pytest

from gpu_util import gpu_ok

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import numpy as np
import torch
import synth
import block_scaled_fp4_nvfp4_amd as m
from gpu_util import dev, dev_bf16, gpu_layer, host

results = []
for w_fmt, a_fmt, tokens in (("nvfp4", "nvfp4", 64), ("mxfp4", "mxfp8", 600)):
    cfg = synth.CONFIGS["tiny"].replace(w_fmt=w_fmt, a_fmt=a_fmt, tokens=tokens, input_seed=7,
                                        shared_inter=128 if a_fmt == "nvfp4" else 0)
    w13, w2 = synth.layer_weights(cfg)
    layer = gpu_layer(cfg, w13, w2, shared=synth.shared_expert(cfg) if cfg.shared_inter else None)
    x = dev_bf16(synth.activations(cfg))
    ids, wts = (dev(a) for a in synth.routing(cfg))
    ws = torch.zeros(m.workspace_size(layer, cfg.tokens), dtype=torch.uint8, device="cuda")
    y = torch.empty(cfg.tokens, cfg.hidden, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print(f"[case] capture first: {{w_fmt}} x {{a_fmt}}, {{tokens}} tokens", flush=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.moe_forward(layer, x, ids, wts, ws, y)
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        outs.append(host(y).copy())
        y.fill_(7.0)
        torch.cuda.synchronize()
    ref = host(m.moe_forward(layer, x, ids, wts))
    for o in outs:
        assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))
    results.append(float(np.abs(ref).max()))
print("CAPTURE_FIRST_OK", results, flush=True)
"""


def test_graph_capture_before_any_eager_forward():
    script = SCRIPT.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(r.stdout[-2000:])
    print(r.stderr[-2000:])
    assert r.returncode == 0 and "CAPTURE_FIRST_OK" in r.stdout
