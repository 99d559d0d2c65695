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


def _check_mxfp8_h(ws, lay, P, I, rows, ref, h, rel=1e-4):
    """MXFP4 x MXFP8 with I a multiple of 128: h leaves the gate_up GEMM's
    epilogue as MXFP8 codes and scales (no f32 h).  The GPU's sorted rows
    `rows` against the oracle's quantization `ref` of its own float64 h (same
    row order).  That h differs from the GPU's f32 h by the MFMA's
    accumulation rounding, whose size follows the row's products rather than
    each value (measured: within 1e-5 of the block amax); so every block
    exponent equal except where the oracle's block amax / 448 lies within
    `rel` of a power of two, and every code equal except, in blocks of equal
    exponent, adjacent codes whose midpoint lies within `rel` times the block
    amax of the oracle's value."""
    from oracle.formats import E4M3_MAX, e4m3_decode
    codes = host(ws[lay["hq_codes"]:lay["hq_codes"] + P * I]).reshape(P, I)[rows].astype(np.int64)
    scales = host(ws[lay["hq_scales"]:lay["hq_scales"] + P * I // 32]).reshape(P, I // 32)[rows].astype(np.int64)
    ref_c = ref["codes"].astype(np.int64)
    ref_s = ref["scales"].astype(np.int64)
    n = len(rows)
    # exponents
    ds = scales != ref_s
    amax = np.abs(h).reshape(n, I // 32, 32).max(axis=2) / E4M3_MAX
    l2 = np.log2(np.where(amax > 0, amax, 1.0))
    assert np.all(np.abs(l2 - np.round(l2))[ds] < 2 * rel / np.log(2)), \
        "exponent differs away from a power-of-two boundary"
    print(f"h blocks with another exponent: {int(ds.sum())} of {ds.size}")
    # codes, in blocks of equal exponent
    same = np.repeat(~ds, 32, axis=1)
    zero = ((codes & 0x7F) == 0) & ((ref_c & 0x7F) == 0)  # +0 / -0: h within rounding of zero
    dc = (codes != ref_c) & same & ~zero
    sign = lambda c: np.where(c & 0x80, -1.0, 1.0)
    vg = sign(codes) * e4m3_decode(codes & 0x7F)
    vr = sign(ref_c) * e4m3_decode(ref_c & 0x7F)
    unit = np.ldexp(1.0, np.repeat(ref_s - 127, 32, axis=1))
    q = h / unit
    mid = (vg + vr) / 2
    bound = rel * np.repeat(amax * E4M3_MAX, 32, axis=1) / unit
    assert np.all(np.abs((codes & 0x7F) - (ref_c & 0x7F))[dc] == 1), "codes differ by more than one step"
    assert np.all(np.abs(q - mid)[dc] <= bound[dc]), "codes differ away from a rounding tie"
    print(f"h codes differing at a tie: {int(dc.sum())} of {dc.size}")
    assert dc.sum() <= 1e-3 * dc.size


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
    P = cfg.pairs
    _, por, _ = moe.permute(ids, cfg.num_experts)
    if a_fmt == "mxfp8":
        _check_mxfp8_h(ws, lay, P, cfg.inter, np.arange(P), {k_: v[por] for k_, v in st["hrec"].items()},
                       st["h"][por])
        return
    # stage: h before its quantization, sorted rows
    h = host(ws[lay["h"]:lay["h"] + 4 * P * cfg.inter].view(torch.float32)).reshape(P, cfg.inter)
    # fp16 MFMA products and sums of exact values: ~1e-7; the block-scaled FP8
    # MFMA accumulates with ~1e-5 relative error (measured)
    assert rel_fro(h, st["h"][por]) < (1e-5 if a_fmt == "nvfp4" else 1e-4)
    if a_fmt == "nvfp4":
        sx = host(ws[lay["x_tensor_scale"]:lay["x_tensor_scale"] + 4].view(torch.float32))[0]
        assert sx == st["xrec"]["tensor_scale"]
        _check_h_tensor_scale(ws, lay, h)


def _ulp16(v):
    """Spacing of fp16 values at |v| (the subnormal spacing 2^-24 below 2^-14)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a >= 2.0 ** -14, a, 1.0)))
    return np.where(a >= 2.0 ** -14, 2.0 ** (e - 10), 2.0 ** -24)


@pytest.mark.parametrize("w_fmt,a_fmt", MODES)
def test_tiny_o_is_the_fp16_rounding_of_the_down_product(tiny, w_fmt, a_fmt):
    """The grouped path holds each pair's unweighted down output o in fp16:
    every o value lies within half an fp16 spacing (plus the f32
    accumulation's rounding) of the float64 product of the GPU's own
    quantized h, dequantized by the oracle, with the oracle's W2 of the
    row's expert.  This isolates the down GEMM and its fp16 store from the
    stages before it.  520 tokens at top-2 (1040 pairs) keep MXFP4 x MXFP8
    off the GEMV path, which takes up to 1024 pairs and keeps o in f32."""
    from oracle import quant as Q
    from oracle.formats import unpack_nibbles
    print_case(f"tiny {w_fmt} x {a_fmt}: o in fp16")
    cfg, w13, w2, _, _, _ = tiny
    cfg = cfg.replace(w_fmt=w_fmt, a_fmt=a_fmt, tokens=520, input_seed=53)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    _, ws, lay = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    P, I, H = cfg.pairs, cfg.inter, cfg.hidden
    assert P > 1024
    offsets, _, _ = moe.permute(ids, cfg.num_experts)
    codes = host(ws[lay["hq_codes"]:lay["hq_codes"] + P * I])
    if a_fmt == "nvfp4":
        sc = host(ws[lay["hq_scales"]:lay["hq_scales"] + P * I // 16]).reshape(P, I // 16)
        sh = host(ws[lay["h_tensor_scale"]:lay["h_tensor_scale"] + 4].view(torch.float32))[0]
        hq = Q.dequantize_nvfp4(unpack_nibbles(codes[:P * I // 2].reshape(P, I // 2)), sc, sh)
    elif a_fmt == "mxfp8":
        sc = host(ws[lay["hq_scales"]:lay["hq_scales"] + P * I // 32]).reshape(P, I // 32)
        hq = Q.dequantize_mxfp8(codes.reshape(P, I), sc)
    else:
        sc = host(ws[lay["hq_scales"]:lay["hq_scales"] + 4 * P * I // 128].view(torch.float32))
        hq = Q.dequantize_fp8_rows(codes.reshape(P, I), sc.reshape(P, I // 128))
    o = host(ws[lay["o"]:lay["o"] + 2 * P * H].view(torch.float16)).astype(np.float64).reshape(P, H)
    ol = OracleLayer(cfg, w13, w2)
    o_ref = np.zeros((P, H))
    for e in range(cfg.num_experts):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            o_ref[r0:r1] = hq[r0:r1] @ moe.dequantize_weight(ol.w2(e), w_fmt).T
    assert np.all(np.isfinite(o))
    # the MFMA's accumulation: fp16 MFMA on exactly decoded values sums exact
    # products in f32 (within 1e-5 of the row's largest value here); the
    # block-scaled FP8 MFMA's sum is less exact (the h stage above allows
    # 1e-4; measured up to about 4e-5 of the row's largest value per element
    # in the MXFP4 x MXFP8 down GEMM)
    slack = (2e-5 if a_fmt == "nvfp4" else 1e-4) * np.abs(o_ref).max(axis=1, keepdims=True)
    bound = 0.5 * _ulp16(np.maximum(np.abs(o_ref), np.abs(o))) + slack
    worst = np.max(np.abs(o - o_ref) / bound)
    print(f"largest |o - o_ref| / bound {worst:.3f}; relative Frobenius {rel_fro(o, o_ref):.3e}")
    assert worst <= 1.0


def _check_h_tensor_scale(ws, lay, h):
    """S_h = fp32(amax / 2688) over the GPU's own f32 h, exactly (the amax
    comes from partial maxima left by the gate_up workgroups)."""
    sh = host(ws[lay["h_tensor_scale"]:lay["h_tensor_scale"] + 4].view(torch.float32))[0]
    assert sh == np.float32(np.float64(np.abs(h).max()) / 2688.0)


def test_tile_weights_layout():
    """moe_fp4_tile_weights only moves bytes: against the same rearrangement
    done in numpy, on random bytes (codes [E][rows/16][K steps][16][64],
    scales [E][rows/16][K steps][16][4])."""
    import block_scaled_fp4_nvfp4_amd as m
    print_case("tile_weights layout")
    rng = np.random.default_rng(7)
    E, rows, cols = 3, 48, 384
    KS = cols // 128
    codes = rng.integers(0, 256, (E, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (E, rows, cols // 32), dtype=np.uint8)
    tc, ts = m.tile_weights(dev(codes), dev(scales))
    torch.cuda.synchronize()
    want_c = codes.reshape(E, rows // 16, 16, KS, 64).transpose(0, 1, 3, 2, 4).reshape(E, rows, cols // 2)
    want_s = scales.reshape(E, rows // 16, 16, KS, 4).transpose(0, 1, 3, 2, 4).reshape(E, rows, cols // 32)
    np.testing.assert_array_equal(host(tc), want_c)
    np.testing.assert_array_equal(host(ts), want_s)
    # NVFP4: the same code order, 8 E4M3 scale bytes per row and step
    scales16 = rng.integers(0, 256, (E, rows, cols // 16), dtype=np.uint8)
    tcn, tsn = m.tile_weights(dev(codes), dev(scales16), "nvfp4")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(tcn), want_c)
    want16 = scales16.reshape(E, rows // 16, 16, KS, 8).transpose(0, 1, 3, 2, 4).reshape(E, rows, cols // 16)
    np.testing.assert_array_equal(host(tsn), want16)
    # block FP8: E4M3 rows of 128 bytes per K step, as two kilobyte halves; no scales
    codes8 = rng.integers(0, 256, (E, rows, cols), dtype=np.uint8)
    tc8, ts8 = m.tile_weights(dev(codes8), None, "fp8_block")
    torch.cuda.synchronize()
    assert ts8 is None
    want8 = codes8.reshape(E, rows // 16, 16, KS, 2, 64).transpose(0, 1, 3, 4, 2, 5).reshape(E, rows, cols)
    np.testing.assert_array_equal(host(tc8), want8)


def _same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def _tile(layer):
    import block_scaled_fp4_nvfp4_amd as m
    f = layer.w_fmt
    layer.w13_tiled, layer.w13_scale_tiled = m.tile_weights(layer.w13, layer.w13_scale, f)
    layer.w2_tiled, layer.w2_scale_tiled = m.tile_weights(layer.w2, layer.w2_scale, f)


@pytest.mark.parametrize("w_fmt,a_fmt", MODES)
def test_tiny_tiled_weights_bit_identical(tiny, w_fmt, a_fmt):
    """With tiled copies of W13 and W2 a GEMM reads the same bytes in another
    order and computes the same sums, so y is bit-identical to the row-major
    layer's.  At these sizes the NVFP4 GEMMs and the MX gate_up take the
    tiled copies; the other GEMMs fall back to the row-major tensors."""
    print_case(f"tiny {w_fmt} x {a_fmt}, tiled weights")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(w_fmt=w_fmt, a_fmt=a_fmt)
    layer = gpu_layer(cfg, w13, w2)
    y0, _, _ = _run(layer, x, ids, wts)
    _tile(layer)
    y1, _, _ = _run(layer, x, ids, wts)
    assert _same_bits(y0, y1)


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


def test_shared_expert_at_model_width():
    """The MXFP8 shared expert at the model's widths (hidden 2560, shared
    1280; the tiny-layer test covers 256 and 128) over 200 tokens (three full
    64-row tiles and a ragged one), next to four NVFP4 routed experts: y
    against the oracle, and the shared part alone (y with it minus y without
    it) against the oracle's."""
    print_case("shared expert at hidden 2560, width 1280, 200 tokens")
    cfg = synth.CONFIGS["prefill_nvfp4"].replace(num_experts=4, top_k=2, tokens=200, input_seed=11)
    assert cfg.shared_inter == 1280 and cfg.hidden == 2560
    w13, w2 = synth.layer_weights(cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    shared = synth.shared_expert(cfg)
    y, _, _ = _run(gpu_layer(cfg, w13, w2, shared=shared), x, ids, wts)
    y0, _, _ = _run(gpu_layer(cfg.replace(shared_inter=0), w13, w2), x, ids, wts)
    ref = OracleLayer(cfg, w13, w2, shared=shared)
    y_ref = moe.moe_forward(ref.as_dict(), x, ids, wts)
    ref0 = ref.as_dict()
    del ref0["shared"]
    y0_ref = moe.moe_forward(ref0, x, ids, wts)
    err, err_s = rel_fro(y, y_ref), rel_fro(y.astype(np.float64) - y0, y_ref - y0_ref)
    print(f"relative Frobenius error: y {err:.3e}, shared part {err_s:.3e}")
    assert err <= TOL and err_s <= TOL
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
    layer = gpu_layer(cfg, w13, w2, shared=synth.shared_expert(cfg))
    y, ws, lay = _run(layer, x, ids, wts)
    sx = host(ws[lay["x_tensor_scale"]:lay["x_tensor_scale"] + 4].view(torch.float32))[0]
    assert sx == gold["s_x"]          # amax/2688 over all of x: exact
    sh = host(ws[lay["h_tensor_scale"]:lay["h_tensor_scale"] + 4].view(torch.float32))[0]
    assert abs(sh / gold["s_h"] - 1) < 1e-5
    P, I = cfg.pairs, cfg.inter
    _check_h_tensor_scale(ws, lay, host(ws[lay["h"]:lay["h"] + 4 * P * I].view(torch.float32)))
    err = rel_fro(y[gold["sample"]], gold["y"])
    print(f"relative Frobenius error on sampled tokens {err:.3e}")
    assert err <= TOL
    assert np.all(np.isfinite(y))
    # tiled copies of W13 and W2 (the benchmark's layer): the whole y bit-identical
    _tile(layer)
    del ws
    y1, _, _ = _run(layer, x, ids, wts)
    assert _same_bits(y, y1)


@pytest.mark.parametrize("name", ["prefill_mxfp4", "prefill_fp8"])
def test_prefill_full_size_sampled(prefill_weights, name):
    """8192 tokens, top-10: MXFP4 x MXFP8 and the block-FP8 copy; the oracle
    computes sampled tokens directly (no whole-tensor activation scale)."""
    print_case(f"{name} full size")
    cfg = synth.CONFIGS[name]
    w13, w2 = prefill_weights  # same bf16 source weights (shared seed)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    layer = gpu_layer(cfg, w13, w2)
    y, ws, lay = _run(layer, x, ids, wts)
    sample = [0, 4095, 8191]
    y_ref, st = moe.moe_forward(OracleLayer(cfg, w13, w2).as_dict(), x, ids, wts, sample_tokens=sample,
                                return_stages=True)
    err = rel_fro(y[sample], y_ref)
    print(f"relative Frobenius error on sampled tokens {err:.3e}")
    assert err <= TOL
    if cfg.a_fmt == "mxfp8" and cfg.inter % 128 == 0:
        # h of the sampled tokens' pairs, quantized in the gate_up epilogue
        k = cfg.top_k
        pairs = np.concatenate([np.arange(t * k, (t + 1) * k) for t in sample])
        _, _, rop = moe.permute(ids, cfg.num_experts)
        _check_mxfp8_h(ws, lay, cfg.pairs, cfg.inter, rop[pairs], st["hrec"], st["h"][pairs])
    # tiled copies of W13 and W2 (the benchmark's prefill layers; both GEMMs
    # read them at these sizes): the whole y bit-identical
    _tile(layer)
    del ws
    y1, _, _ = _run(layer, x, ids, wts)
    assert _same_bits(y, y1)
