"""Pins of the oracle MoE layer: permutation by brute force, reduction to a
dense SwiGLU, invariances (expert relabeling, routing-weight scaling, zero
padding: "silu(0) * 0 = 0", FP4-Local AZ card, section "The shared expert"),
and the quantization-error sanity band (QAD5500-Hybrid card, "Verification":
a quantized copy differs by a few percent, an unrelated one by ~100 %)."""
import math

import numpy as np
import pytest

import synth
from oracle import moe, quant
from oracle.formats import bf16_to_f64, bf16_bits_from_f32


def _layer(cfg, w13_bits, w2_bits, w_fmt=None, a_fmt=None, rule="4over6"):
    w_fmt = w_fmt or cfg.w_fmt
    a_fmt = a_fmt or cfg.a_fmt
    q13 = [moe.quantize_expert_weight(w, w_fmt, rule) for w in w13_bits]
    q2 = [moe.quantize_expert_weight(w, w_fmt, rule) for w in w2_bits]
    return dict(w_fmt=w_fmt, a_fmt=a_fmt, num_experts=len(q13), hidden=w13_bits.shape[2],
                inter=w13_bits.shape[1] // 2, w13=lambda e: q13[e], w2=lambda e: q2[e]), q13, q2


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w13, w2 = synth.layer_weights(cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    return cfg, w13, w2, x, ids, wts


def test_permutation_brute_force():
    rng = np.random.default_rng(0)
    for T, k, E in [(64, 2, 8), (16, 10, 512), (5, 3, 4), (0, 2, 4)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]) if T else np.zeros((0, k), int)
        off, por, rop = moe.permute(ids, E)
        rows = []
        for e in range(E):
            mine = [p for p in range(T * k) if ids.reshape(-1)[p] == e]
            assert off[e + 1] - off[e] == len(mine)
            rows += mine
        np.testing.assert_array_equal(por, rows)
        assert off[-1] == T * k and sorted(por.tolist()) == list(range(T * k))
        np.testing.assert_array_equal(por[rop], np.arange(T * k))


def test_router_topk_renormalized():
    cfg = synth.CONFIGS["tiny"]
    ids, w = synth.routing(cfg)
    lg = synth.router_logits(cfg)
    for t in range(cfg.tokens):
        top = sorted(range(cfg.num_experts), key=lambda e: (-lg[t, e], e))[:cfg.top_k]
        assert list(ids[t]) == top
        z = np.exp(lg[t, top].astype(np.float64) - lg[t, top].max())
        np.testing.assert_allclose(w[t], z / z.sum(), rtol=1e-6)
    assert np.all(np.abs(w.sum(1) - 1) < 1e-6)


def test_single_expert_reduces_to_dense_swiglu(tiny):
    cfg, w13, w2, x, _, _ = tiny
    layer, q13, q2 = _layer(cfg, w13[:1], w2[:1])
    ids = np.zeros((cfg.tokens, 1), np.int32)
    wts = np.ones((cfg.tokens, 1), np.float32)
    y = moe.moe_forward(layer, x, ids, wts)
    W13 = quant.dequantize_nvfp4(q13[0]["codes"], q13[0]["scales"], q13[0]["tensor_scale"])
    W2 = quant.dequantize_nvfp4(q2[0]["codes"], q2[0]["scales"], q2[0]["tensor_scale"])
    xf = bf16_to_f64(x)
    I = cfg.inter
    g, u = xf @ W13[:I].T, xf @ W13[I:].T
    ref = ((g / (1 + np.exp(-g))) * u) @ W2.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_relabel_and_weight_scaling(tiny):
    cfg, w13, w2, x, ids, wts = tiny
    layer, _, _ = _layer(cfg, w13, w2)
    y = moe.moe_forward(layer, x, ids, wts)
    perm = np.random.default_rng(1).permutation(cfg.num_experts)   # new id of old expert e
    inv = np.argsort(perm)
    layer2, _, _ = _layer(cfg, w13[inv], w2[inv])
    np.testing.assert_array_equal(moe.moe_forward(layer2, x, perm[ids], wts), y)
    np.testing.assert_array_equal(moe.moe_forward(layer, x, ids, 2 * wts), 2 * y)


def test_zero_padding_is_output_invariant(tiny):
    cfg, w13, w2, x, ids, wts = tiny
    I, pad = cfg.inter, 32
    z = np.zeros((w13.shape[0], pad, w13.shape[2]), np.uint16)
    w13p = np.concatenate([w13[:, :I], z, w13[:, I:], z], axis=1)
    w2p = np.concatenate([w2, np.zeros((w2.shape[0], w2.shape[1], pad), np.uint16)], axis=2)
    for a_fmt in ("none", "nvfp4"):
        layer, q13, _ = _layer(cfg, w13, w2, a_fmt=a_fmt)
        layerp, q13p, _ = _layer(cfg.replace(inter=I + pad), w13p, w2p, a_fmt=a_fmt)
        assert q13p[0]["tensor_scale"] == q13[0]["tensor_scale"]
        y = moe.moe_forward(layer, x, ids, wts)
        yp = moe.moe_forward(layerp, x, ids, wts)
        # identical up to float64 summation order of the matmul library
        np.testing.assert_allclose(yp, y, rtol=1e-12, atol=1e-14)


def test_activation_tensor_scale_is_amax_over_2688(tiny):
    cfg, w13, w2, x, ids, wts = tiny
    layer, _, _ = _layer(cfg, w13, w2, a_fmt="nvfp4")
    _, st = moe.moe_forward(layer, x, ids, wts, return_stages=True)
    xf = bf16_to_f64(x)
    assert st["xrec"]["tensor_scale"] == np.float32(np.max(np.abs(xf)) / 2688.0)
    assert st["hrec"]["tensor_scale"] == np.float32(np.max(np.abs(st["h"])) / 2688.0)
    # the M=6 plan maps each tensor's max block to scale byte 0x7E
    assert 0x7E in st["xrec"]["scales"] and not st["xrec"]["m4"].any()


@pytest.mark.parametrize("w_fmt,a_fmt", [("nvfp4", "none"), ("nvfp4", "nvfp4"),
                                         ("mxfp4", "mxfp8"), ("fp8_block", "fp8_row")])
def test_quantized_layer_differs_by_a_plausible_amount(tiny, w_fmt, a_fmt):
    cfg, w13, w2, x, ids, wts = tiny
    layer, _, _ = _layer(cfg, w13, w2, w_fmt=w_fmt, a_fmt=a_fmt)
    y = moe.moe_forward(layer, x, ids, wts)
    xf = bf16_to_f64(x)
    ref = np.zeros_like(y)
    for t in range(cfg.tokens):
        for j in range(cfg.top_k):
            e = ids[t, j]
            ref[t] += wts[t, j] * moe.dense_swiglu(xf[t:t + 1], bf16_to_f64(w13[e]), bf16_to_f64(w2[e]))[0]
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    lo, hi = (0.005, 0.08) if w_fmt == "fp8_block" else (0.01, 0.3)
    assert lo < rel < hi, rel


def test_sampled_tokens_match_full_forward(tiny):
    cfg, w13, w2, x, ids, wts = tiny
    for a_fmt in ("none", "nvfp4"):
        layer, _, _ = _layer(cfg, w13, w2, a_fmt=a_fmt)
        y = moe.moe_forward(layer, x, ids, wts)
        ys = moe.moe_forward(layer, x, ids, wts, sample_tokens=[3, 40, 63])
        np.testing.assert_allclose(ys, y[[3, 40, 63]], rtol=1e-12, atol=1e-15)


def test_shared_expert_gate_and_band():
    rng = np.random.default_rng(2)
    H, S, T = 256, 128, 16
    xb = bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    w13 = bf16_bits_from_f32((rng.standard_normal((2 * S, H)) * 0.02).astype(np.float32))
    w2 = bf16_bits_from_f32((rng.standard_normal((H, S)) * 0.02).astype(np.float32))
    wg = bf16_bits_from_f32((rng.standard_normal(H) * 0.02).astype(np.float32))
    sh = dict(w13=moe.quantize_expert_weight(w13, "mxfp8"), w2=moe.quantize_expert_weight(w2, "mxfp8"),
              gate_bits=wg)
    x = bf16_to_f64(xb)
    out = moe.shared_forward(sh, x)
    gate = 1 / (1 + np.exp(-(x @ bf16_to_f64(wg))))
    ref = gate[:, None] * moe.dense_swiglu(x, bf16_to_f64(w13), bf16_to_f64(w2))
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 0.01 < rel < 0.1, rel
    # zero gate vector -> sigmoid(0) = 1/2 exactly
    sh0 = dict(sh, gate_bits=np.zeros(H, np.uint16))
    g0 = moe.shared_forward(sh0, x)
    np.testing.assert_array_equal(2 * g0, moe.shared_forward(dict(sh0), x) * 2)
    np.testing.assert_allclose(g0 / out, (0.5 / gate)[:, None] * np.ones_like(out), rtol=1e-12)


# ------------------------------------------------ activation functions
# The shared expert's gate is a sigmoid and every expert's gate activation is
# SiLU (FP4-Local AZ card, "The shared expert").  Pinned by identities and
# closed-form values of the functions, not by restating their formulas.

def _sigmoid_pins_hold(f):
    v = np.linspace(-30.0, 30.0, 601)
    ok = np.allclose(f(v) + f(-v), 1.0, rtol=0, atol=1e-15)          # symmetry
    ok &= abs(f(np.float64(math.log(3.0))) - 0.75) < 1e-15           # e^-ln3 = 1/3 -> 1/(1+1/3)
    ok &= f(np.float64(0.0)) == 0.5
    ok &= bool(np.all(np.diff(f(v)) > 0))                            # increasing
    ok &= 0.0 < f(np.float64(-40.0)) < 1e-17                         # ~ e^-40 = 4.25e-18
    ok &= f(np.float64(40.0)) == 1.0
    return bool(ok)


def _silu_pins_hold(f):
    v = np.linspace(-30.0, 30.0, 601)
    ok = np.allclose(f(v) - f(-v), v, rtol=0, atol=1e-13)             # silu(v) - silu(-v) = v
    ok &= abs(f(np.float64(math.log(3.0))) - 0.75 * math.log(3.0)) < 1e-15
    ok &= f(np.float64(0.0)) == 0.0
    ok &= -1e-15 < f(np.float64(-40.0)) < 0.0                        # ~ -40 e^-40
    ok &= f(np.float64(40.0)) == 40.0
    # minimum near v = -1.2785 (root of 1 + v (1 - sigmoid(v)) = 0), value -0.27846
    ok &= abs(float(np.min(f(np.linspace(-3, 0, 30001)))) + 0.278464542761074) < 1e-9
    return bool(ok)


def test_sigmoid_closed_forms():
    assert _sigmoid_pins_hold(moe.sigmoid)
    # planted mistakes each fail: sign flip, the complement, a doubled slope
    assert not _sigmoid_pins_hold(lambda v: 1.0 / (1.0 + np.exp(v)))
    assert not _sigmoid_pins_hold(lambda v: np.exp(-v) / (1.0 + np.exp(-v)))
    assert not _sigmoid_pins_hold(lambda v: 1.0 / (1.0 + np.exp(-2.0 * v)))


def test_silu_closed_forms():
    assert _silu_pins_hold(moe.silu)
    assert not _silu_pins_hold(lambda v: v / (1.0 + np.exp(v)))           # sign flip
    assert not _silu_pins_hold(lambda v: v / (1.0 + np.exp(-2.0 * v)))    # doubled slope
    assert not _silu_pins_hold(lambda v: 1.0 / (1.0 + np.exp(-v)))        # the sigmoid alone
    assert not _silu_pins_hold(lambda v: np.maximum(v, 0.0))              # ReLU


# ----------------------------------------------------------------- routing

def test_route_hand_example_and_ties():
    # l' = [0, ln 2, 0, -1]: ln 2 first, then the tie at 0 goes to the lower id;
    # weights e^(ln2)/(e^(ln2)+1) = 2/3 and 1/3 (ln 2 rounded to f32 moves them < 1e-7)
    lg = np.array([[0.0, math.log(2.0), 0.0, -1.0]], np.float32)
    ids, w = moe.route(lg, None, 2)
    assert ids.tolist() == [[1, 0]]
    np.testing.assert_allclose(w[0], [2 / 3, 1 / 3], rtol=2e-7)
    # all equal: k = E keeps id order and weights 1/E
    ids, w = moe.route(np.zeros((2, 8), np.float32), None, 8)
    assert ids.tolist() == [list(range(8))] * 2
    assert np.all(w == np.float32(1 / 8))


def test_route_bias_and_invariants():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((64, 40)).astype(np.float32)
    bias = np.zeros(40, np.float32)
    bias[17] = 100.0
    ids, w = moe.route(lg, bias, 5)
    assert np.all(ids[:, 0] == 17) and np.all(w[:, 0] > 0.99)
    ids, w = moe.route(lg, None, 6)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, rtol=0, atol=3e-7)
    assert np.all(np.diff(w, axis=1) <= 0)                       # weights follow the logit order
    sel = np.take_along_axis(lg, ids, axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    assert np.all(np.sort(lg, axis=1)[:, -6][:, None] <= sel)    # the k largest
    # relabeling experts relabels the ids and leaves the weights
    perm = rng.permutation(40)
    ids2, w2 = moe.route(lg[:, np.argsort(perm)], None, 6)
    np.testing.assert_array_equal(np.argsort(perm)[ids2], ids)   # no ties in continuous data
    np.testing.assert_array_equal(w2, w)
    # the first k' of a top-k selection are the top-k' selection
    ids3, _ = moe.route(lg, None, 3)
    np.testing.assert_array_equal(ids3, ids[:, :3])


def test_route_agrees_with_the_input_generator():
    """synth.route writes the same reading with numpy's stable argsort and a
    plain float64 sum: selections must be identical, weights within 1 ulp."""
    cfg = synth.CONFIGS["prefill_nvfp4"].replace(tokens=256)
    lg, b = synth.router_logits(cfg), synth.router_bias(cfg)
    a_ids, a_w = moe.route(lg, b, cfg.top_k)
    s_ids, s_w = synth.route(lg, b, cfg.top_k)
    np.testing.assert_array_equal(a_ids, s_ids)
    np.testing.assert_array_max_ulp(a_w, s_w, maxulp=1)
