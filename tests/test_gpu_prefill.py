"""GPU parity of the quantized-activation MoE paths (grouped MFMA GEMMs):
NVFP4 W4A4, MXFP4 x MXFP8, block FP8, and the MXFP8 shared expert, against
the float64 oracle.  Bar: relative Frobenius error <= 2e-3 on y."""
import numpy as np
import pytest

import synth
from oracle import moe

from gpu_util import (OracleLayer, dev, dev_bf16, gpu_layer, gpu_ok, host, print_case,
                      rel_fro, torch)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

TOL = 2e-3
MODES = [("nvfp4", "nvfp4"), ("mxfp4", "mxfp8"), ("fp8_block", "fp8_row")]


def _run(layer, x_bits, ids, wts):
    import block_scaled_fp4_nvfp4_amd as m
    T = x_bits.shape[0]
    ws = torch.zeros(m.workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    y = m.moe_forward(layer, dev_bf16(x_bits), dev(ids.astype(np.int32)), dev(wts.astype(np.float32)), ws)
    torch.cuda.synchronize()
    return host(y), ws, m.workspace_layout(layer, T)


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w13, w2 = synth.layer_weights(cfg)
    return cfg, w13, w2, synth.activations(cfg), *synth.routing(cfg)


@pytest.mark.parametrize("w_fmt,a_fmt", MODES)
def test_tiny_quantized_activations(tiny, w_fmt, a_fmt):
    print_case(f"tiny {w_fmt} x {a_fmt}")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(w_fmt=w_fmt, a_fmt=a_fmt)
    y, ws, lay = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    ol = OracleLayer(cfg, w13, w2)
    y_ref, st = moe.moe_forward(ol.as_dict(), x, ids, wts, return_stages=True)
    err = rel_fro(y, y_ref)
    print(f"relative Frobenius error {err:.3e}")
    assert err <= TOL
    # stage: h before its quantization, sorted rows
    P = cfg.pairs
    _, por, _ = moe.permute(ids, cfg.num_experts)
    h = host(ws[lay["h"]:lay["h"] + 4 * P * cfg.inter].view(torch.float32)).reshape(P, cfg.inter)
    # fp16 MFMA products and sums of exact values: ~1e-7; the block-scaled FP8
    # MFMA accumulates its 128 products with ~1e-5 relative error (measured)
    assert rel_fro(h, st["h"][por]) < (1e-5 if a_fmt == "nvfp4" else 1e-4)
    if a_fmt == "nvfp4":
        sx = host(ws[lay["x_tensor_scale"]:lay["x_tensor_scale"] + 4].view(torch.float32))[0]
        assert sx == st["xrec"]["tensor_scale"]


def test_tiny_w4a4_static_scales(tiny):
    """Static input_scale / intermediate scale (calibrated export, Local-Hessian card)."""
    print_case("tiny W4A4 static scales")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(a_fmt="nvfp4")
    layer = gpu_layer(cfg, w13, w2)
    sx, sh = np.float32(0.0021), np.float32(0.00011)
    layer.input_scale = torch.tensor([sx], device="cuda")
    layer.inter_scale = torch.tensor([sh], device="cuda")
    y, _, _ = _run(layer, x, ids, wts)
    from oracle import quant
    from oracle.formats import bf16_to_f64
    ol = OracleLayer(cfg, w13, w2)
    # oracle with the same static scales: quantize x and h with the given tensor scales
    orig = moe.quantize_activation

    def static_q(v, a_fmt, _state={"n": 0}):
        if a_fmt != "nvfp4":
            return orig(v, a_fmt)
        s = sx if _state["n"] == 0 else sh
        _state["n"] += 1
        q = quant.quantize_nvfp4(v, "rtn", tensor_scale=s)
        return quant.dequantize_nvfp4(q["codes"], q["scales"], q["tensor_scale"]), q
    moe.quantize_activation = static_q
    try:
        y_ref = moe.moe_forward(ol.as_dict(), x, ids, wts)
    finally:
        moe.quantize_activation = orig
    assert rel_fro(y, y_ref) <= TOL


@pytest.mark.parametrize("w_fmt,a_fmt", MODES)
def test_tiny_zero_padding_bit_identical(tiny, w_fmt, a_fmt):
    print_case(f"tiny zero padding {w_fmt}")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(w_fmt=w_fmt, a_fmt=a_fmt)
    I, pad = cfg.inter, 128
    z = np.zeros((w13.shape[0], pad, w13.shape[2]), np.uint16)
    w13p = np.concatenate([w13[:, :I], z, w13[:, I:], z], axis=1)
    w2p = np.concatenate([w2, np.zeros((w2.shape[0], w2.shape[1], pad), np.uint16)], axis=2)
    y, _, _ = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    yp, _, _ = _run(gpu_layer(cfg.replace(inter=I + pad), w13p, w2p), x, ids, wts)
    np.testing.assert_array_equal(y.view(np.uint32), yp.view(np.uint32))


def test_tiny_shared_expert(tiny):
    print_case("tiny W4A4 + MXFP8 shared expert")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(a_fmt="nvfp4", shared_inter=128)
    shared = synth.shared_expert(cfg)
    y, _, _ = _run(gpu_layer(cfg, w13, w2, shared=shared), x, ids, wts)
    y_ref = moe.moe_forward(OracleLayer(cfg, w13, w2, shared=shared).as_dict(), x, ids, wts)
    assert rel_fro(y, y_ref) <= TOL
    # the shared contribution is actually there
    y0, _, _ = _run(gpu_layer(cfg.replace(shared_inter=0), w13, w2), x, ids, wts)
    assert rel_fro(y, y0) > 0.05


def test_tiny_invalid_ids_w4a4(tiny):
    print_case("tiny W4A4 invalid ids")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(a_fmt="nvfp4")
    bad = ids.copy()
    bad[3, 0] = 1000
    y, ws, lay = _run(gpu_layer(cfg, w13, w2), x, bad, wts)
    assert host(ws[lay["error_flag"]:lay["error_flag"] + 4].view(torch.int32))[0] == 1
    assert np.all(np.isfinite(y))


# ------------------------------------------------------------ full-size layers

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden",
                                    "prefill_nvfp4_sampled.npz")


@pytest.fixture(scope="module")
def prefill_weights():
    cfg = synth.CONFIGS["prefill_nvfp4"]
    return synth.layer_weights(cfg)


def test_prefill_nvfp4_full_size_sampled(prefill_weights):
    """8192 tokens, top-5, biased router, NVFP4 W4A4 + MXFP8 shared expert 1280,
    in the benchmark's launch configuration; sampled tokens against the stored
    oracle outputs (tests/golden/make_prefill_golden.py)."""
    print_case("prefill NVFP4 W4A4 full size")
    cfg = synth.CONFIGS["prefill_nvfp4"]
    gold = np.load(GOLDEN)
    w13, w2 = prefill_weights
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    np.testing.assert_array_equal(np.bincount(ids.reshape(-1), minlength=cfg.num_experts), gold["counts"])
    y, ws, lay = _run(gpu_layer(cfg, w13, w2, shared=synth.shared_expert(cfg)), x, ids, wts)
    sx = host(ws[lay["x_tensor_scale"]:lay["x_tensor_scale"] + 4].view(torch.float32))[0]
    assert sx == gold["s_x"]          # amax/2688 over all of x: exact
    sh = host(ws[lay["h_tensor_scale"]:lay["h_tensor_scale"] + 4].view(torch.float32))[0]
    assert abs(sh / gold["s_h"] - 1) < 1e-5
    err = rel_fro(y[gold["sample"]], gold["y"])
    print(f"relative Frobenius error on sampled tokens {err:.3e}")
    assert err <= TOL
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("name", ["prefill_mxfp4", "prefill_fp8"])
def test_prefill_full_size_sampled(prefill_weights, name):
    """8192 tokens, top-10: MXFP4 x MXFP8 and the block-FP8 copy; the oracle
    computes sampled tokens directly (no whole-tensor activation scale)."""
    print_case(f"{name} full size")
    cfg = synth.CONFIGS[name]
    w13, w2 = prefill_weights  # same bf16 source weights (shared seed)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, _, _ = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    sample = [0, 4095, 8191]
    y_ref = moe.moe_forward(OracleLayer(cfg, w13, w2).as_dict(), x, ids, wts, sample_tokens=sample)
    err = rel_fro(y[sample], y_ref)
    print(f"relative Frobenius error on sampled tokens {err:.3e}")
    assert err <= TOL
