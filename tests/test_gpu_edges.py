"""Edge cases of moe_fp4_forward in every operand mode, against the float64
oracle: a single token; every token routed to the same two experts (two
full 64-row tiles and a 2-row tail each, all other experts empty); exactly
1024 pairs (the largest batch of the one-workgroup permutation and of the
MXFP4 x MXFP8 GEMV path); 1026 pairs (the multi-pass permutation, and the
grouped GEMMs for MXFP4 x MXFP8).  Tiny layer: 8 experts, hidden 256,
intermediate 128."""
import numpy as np
import pytest

import synth
from oracle import moe

from gpu_util import OracleLayer, dev, dev_bf16, gpu_layer, gpu_ok, host, print_case, rel_fro, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

TOL = 2e-3
MODES = [("nvfp4", "none"), ("nvfp4", "nvfp4"), ("mxfp4", "mxfp8"), ("fp8_block", "fp8_row")]


@pytest.fixture(scope="module")
def weights():
    cfg = synth.CONFIGS["tiny"]
    return synth.layer_weights(cfg)


def _run(layer, x_bits, ids, wts):
    import block_scaled_fp4_nvfp4_amd as m
    T = x_bits.shape[0]
    ws = torch.zeros(m.workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    y = m.moe_forward(layer, dev_bf16(x_bits), dev(ids.astype(np.int32)), dev(wts.astype(np.float32)), ws)
    torch.cuda.synchronize()
    lay = m.workspace_layout(layer, T)
    flag = int(host(ws[lay["error_flag"]:lay["error_flag"] + 4].view(torch.int32))[0])
    return host(y), flag


def _case(name, cfg):
    """(x bits, ids, weights) of the named routing case."""
    if name == "hot_pair":  # every token to experts 3 and 5
        c = cfg.replace(tokens=130, input_seed=21)
        ids = np.tile(np.array([[3, 5]], np.int32), (c.tokens, 1))
        wts = np.tile(np.array([[0.625, 0.375]], np.float32), (c.tokens, 1))
        return c, synth.activations(c), ids, wts
    tokens = {"single": 1, "pairs_1024": 512, "pairs_1026": 513}[name]
    c = cfg.replace(tokens=tokens, input_seed=22 + tokens)
    ids, wts = synth.routing(c)
    return c, synth.activations(c), ids, wts


@pytest.mark.parametrize("name", ["single", "hot_pair", "pairs_1024", "pairs_1026"])
@pytest.mark.parametrize("w_fmt,a_fmt", MODES)
def test_edge_routing(weights, name, w_fmt, a_fmt):
    print_case(f"edge {name}: {w_fmt} x {a_fmt}")
    w13, w2 = weights
    base = synth.CONFIGS["tiny"].replace(w_fmt=w_fmt, a_fmt=a_fmt, rule="rtn" if w_fmt == "fp8_block" else "4over6")
    cfg, x, ids, wts = _case(name, base)
    y, flag = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    assert flag == 0
    assert np.all(np.isfinite(y))
    y_ref = moe.moe_forward(OracleLayer(cfg, w13, w2).as_dict(), x, ids, wts)
    err = rel_fro(y, y_ref)
    print(f"relative Frobenius error {err:.3e}")
    assert err <= TOL
    if a_fmt == "none":  # bf16 activations: f32 accumulation only
        assert err < 1e-5
    # each token on its own (a token's k rows may sit in any tile): a wrong
    # row would be off by order 1.  With quantized activations one h code
    # flipped at a rounding tie moves a token by up to about a code step of
    # that h element's contribution (measured up to 1.2e-2 with FP8 h, whose
    # steps are 1/8 relative); with bf16 activations only summation order
    # differs
    worst = max(rel_fro(y[t], y_ref[t]) for t in range(cfg.tokens))
    print(f"worst token {worst:.3e}")
    assert worst <= (1e-5 if a_fmt == "none" else 5e-2), worst
