"""GPU MoE forward parity through the C ABI against the float64 oracle.

Bar: relative Frobenius error <= 2e-3 on y; the permutation is compared
exactly; stage-wise checks read the forward's workspace buffers (offsets
from moe_fp4_workspace_layout)."""
import numpy as np
import pytest

import synth
from oracle import moe

from gpu_util import (OracleLayer, dev, dev_bf16, gpu_layer, gpu_ok, host, print_case,
                      rel_fro, torch)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

TOL = 2e-3


def _lib():
    import block_scaled_fp4_nvfp4_amd as m
    return m


def _run(layer, x_bits, ids, wts):
    m = _lib()
    T = x_bits.shape[0]
    ws = torch.zeros(m.workspace_size(layer, T), dtype=torch.uint8, device="cuda")
    y = m.moe_forward(layer, dev_bf16(x_bits), dev(ids.astype(np.int32)), dev(wts.astype(np.float32)), ws)
    torch.cuda.synchronize()
    return host(y), ws, m.workspace_layout(layer, T)


def _ws_i32(ws, off, n):
    return host(ws[off:off + 4 * n].view(torch.int32))


def _ws_f32(ws, off, n):
    return host(ws[off:off + 4 * n].view(torch.float32))


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w13, w2 = synth.layer_weights(cfg)
    return cfg, w13, w2, synth.activations(cfg), *synth.routing(cfg)


@pytest.mark.parametrize("w_fmt", ["nvfp4", "mxfp4"])
def test_tiny_w4a16_matches_oracle(tiny, w_fmt):
    print_case(f"tiny W4A16 {w_fmt}")
    cfg, w13, w2, x, ids, wts = tiny
    cfg = cfg.replace(w_fmt=w_fmt)
    y, ws, lay = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    ol = OracleLayer(cfg, w13, w2)
    y_ref, st = moe.moe_forward(ol.as_dict(), x, ids, wts, return_stages=True)
    assert rel_fro(y, y_ref) <= TOL
    assert rel_fro(y, y_ref) < 1e-5          # f32 accumulation only
    # permutation: exact
    P = cfg.tokens * cfg.top_k
    off, por, rop = moe.permute(ids, cfg.num_experts)
    np.testing.assert_array_equal(_ws_i32(ws, lay["offsets"], cfg.num_experts + 1), off)
    np.testing.assert_array_equal(_ws_i32(ws, lay["pair_of_row"], P), por)
    np.testing.assert_array_equal(_ws_i32(ws, lay["row_of_pair"], P), rop)
    assert _ws_i32(ws, lay["error_flag"], 1)[0] == 0
    # stage: h in sorted row order
    h = _ws_f32(ws, lay["h"], P * cfg.inter).reshape(P, cfg.inter)
    assert rel_fro(h, st["h"][por]) < 1e-5


def test_tiny_zero_padding_bit_identical(tiny):
    """640 real + 640 zero rows give bit-identical output (FP4-Local AZ card,
    "The shared expert": silu(0) * 0 = 0); here 128 -> 160 zero-padded."""
    print_case("tiny zero padding")
    cfg, w13, w2, x, ids, wts = tiny
    I, pad = cfg.inter, 32
    z = np.zeros((w13.shape[0], pad, w13.shape[2]), np.uint16)
    w13p = np.concatenate([w13[:, :I], z, w13[:, I:], z], axis=1)
    w2p = np.concatenate([w2, np.zeros((w2.shape[0], w2.shape[1], pad), np.uint16)], axis=2)
    y, _, _ = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    yp, _, _ = _run(gpu_layer(cfg.replace(inter=I + pad), w13p, w2p), x, ids, wts)
    np.testing.assert_array_equal(y.view(np.uint32), yp.view(np.uint32))


def test_tiny_invalid_ids_flagged_and_skipped(tiny):
    print_case("tiny invalid ids")
    cfg, w13, w2, x, ids, wts = tiny
    bad = ids.copy()
    bad[5, 1] = cfg.num_experts + 3
    bad[9, 0] = -1
    y, ws, lay = _run(gpu_layer(cfg, w13, w2), x, bad, wts)
    assert _ws_i32(ws, lay["error_flag"], 1)[0] == 2
    wz = wts.copy()
    wz[5, 1] = 0.0
    wz[9, 0] = 0.0
    fixed = ids.copy()
    fixed[5, 1] = 0
    fixed[9, 0] = 0
    y_ref = moe.moe_forward(OracleLayer(cfg, w13, w2).as_dict(), x, fixed, wz)
    assert rel_fro(y, y_ref) < 1e-5


def test_tiny_all_ids_invalid_gives_zero(tiny):
    """No pair valid: no expert is active, y is the combine of no rows (zero),
    and the flag counts every pair."""
    print_case("tiny all ids invalid")
    cfg, w13, w2, x, ids, wts = tiny
    bad = np.full_like(ids, cfg.num_experts)
    y, ws, lay = _run(gpu_layer(cfg, w13, w2), x, bad, wts)
    assert _ws_i32(ws, lay["error_flag"], 1)[0] == bad.size
    assert np.all(y == 0.0)


@pytest.mark.parametrize("w_fmt,a_fmt", [("nvfp4", "none"), ("mxfp4", "none"), ("mxfp4", "mxfp8")])
def test_gemv_path_batch_invariant(tiny, w_fmt, a_fmt):
    """The same 16 tokens alone and as the first rows of a 65-token batch give
    bit-identical y: every stage of the GEMV path is per row (per-token MXFP8
    blocks, per-pair dot products in a fixed lane order) and the combine adds
    each token's slots in order, so neither the other tokens nor the grid
    shape reach a token's output."""
    print_case(f"GEMV path batch invariance {w_fmt} x {a_fmt}")
    cfg, w13, w2, _, _, _ = tiny
    c = cfg.replace(w_fmt=w_fmt, a_fmt=a_fmt, tokens=65, input_seed=31)
    x, ids, wts = synth.activations(c), *synth.routing(c)
    layer = gpu_layer(c, w13, w2)
    y65, _, _ = _run(layer, x, ids, wts)
    y16, _, _ = _run(layer, x[:16], ids[:16], wts[:16])
    np.testing.assert_array_equal(y16.view(np.uint32), y65[:16].view(np.uint32))
    y_ref = moe.moe_forward(OracleLayer(c, w13, w2).as_dict(), x, ids, wts)
    assert rel_fro(y65, y_ref) <= TOL


@pytest.mark.parametrize("w_fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("with_shared", [False, True])
def test_gemv_path_permutations_agree(tiny, w_fmt, with_shared):
    """512 tokens at top-2 (1024 pairs: the one-workgroup permutation) and the
    same tokens as the head of a 513-token batch (the multi-pass one) give
    bit-identical y on the bf16-activation GEMV path, with pairs out of range
    (token 3 has no valid pair, so its y is the shared expert's output alone,
    or zero) and with the MXFP8 shared expert added on a second stream; y also
    against the oracle."""
    print_case(f"GEMV path, both permutations {w_fmt}, shared={with_shared}")
    cfg, w13, w2, _, _, _ = tiny
    c = cfg.replace(w_fmt=w_fmt, tokens=513, input_seed=41, shared_inter=128 if with_shared else 0)
    x = synth.activations(c)
    ids, wts = synth.routing(c)
    ids = ids.copy()
    ids[3, :] = c.num_experts
    ids[7, 1] = -1
    ids[400, 0] = c.num_experts + 5
    shared = synth.shared_expert(c) if with_shared else None
    layer = gpu_layer(c, w13, w2, shared=shared)
    y513, _, _ = _run(layer, x, ids, wts)
    y512, ws, lay = _run(layer, x[:512], ids[:512], wts[:512])
    assert _ws_i32(ws, lay["error_flag"], 1)[0] == c.top_k + 2
    np.testing.assert_array_equal(y512.view(np.uint32), y513[:512].view(np.uint32))
    if not with_shared:
        assert np.all(y512[3] == 0.0)
    fixed, wz = ids.copy(), wts.copy()
    bad = (ids < 0) | (ids >= c.num_experts)
    fixed[bad], wz[bad] = 0, 0.0
    y_ref = moe.moe_forward(OracleLayer(c, w13, w2, shared=shared).as_dict(), x[:512], fixed[:512], wz[:512])
    assert rel_fro(y512, y_ref) <= TOL


def test_single_expert_top1_reduces_to_dense(tiny):
    print_case("tiny E=1 k=1")
    cfg, w13, w2, x, _, _ = tiny
    c1 = cfg.replace(num_experts=1, top_k=1)
    ids = np.zeros((cfg.tokens, 1), np.int32)
    wts = np.ones((cfg.tokens, 1), np.float32)
    y, _, _ = _run(gpu_layer(c1, w13[:1], w2[:1]), x, ids, wts)
    ol = OracleLayer(c1, w13[:1], w2[:1])
    from oracle.quant import dequantize_nvfp4
    from oracle.formats import bf16_to_f64
    a, b = ol.w13(0), ol.w2(0)
    W13 = dequantize_nvfp4(a["codes"], a["scales"], a["tensor_scale"])
    W2 = dequantize_nvfp4(b["codes"], b["scales"], b["tensor_scale"])
    ref = moe.dense_swiglu(bf16_to_f64(x), W13, W2)
    assert rel_fro(y, ref) < 1e-5


@pytest.fixture(scope="module")
def decode_layer():
    cfg = synth.CONFIGS["decode"]
    w13, w2 = synth.layer_weights(cfg)
    return cfg, w13, w2


def test_decode_layer_all_tokens(decode_layer):
    """512 experts, top-10, hidden 2560, inter 640, 16 tokens: the workload
    and launch configuration the benchmark times; every token vs the oracle
    (its 134 touched experts quantized by the oracle in a process pool)."""
    print_case("decode layer, all 16 tokens")
    cfg, w13, w2 = decode_layer
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, ws, lay = _run(gpu_layer(cfg, w13, w2), x, ids, wts)
    ol = OracleLayer(cfg, w13, w2)
    ol.prefetch(np.unique(ids))
    y_ref = moe.moe_forward(ol.as_dict(), x, ids, wts)
    err = rel_fro(y, y_ref)
    print(f"relative Frobenius error over all tokens {err:.3e}")
    assert err <= TOL
    assert err < 1e-5
    for t in range(cfg.tokens):  # each token on its own
        assert rel_fro(y[t], y_ref[t]) < 1e-5, t
    off, por, _ = moe.permute(ids, cfg.num_experts)
    np.testing.assert_array_equal(_ws_i32(ws, lay["pair_of_row"], cfg.pairs), por)
    assert np.all(np.isfinite(y)) and np.linalg.norm(y) > 0


def test_decode_layer_graph_replay_bit_identical(decode_layer):
    """The decode layer as the benchmark times it: several forwards of the
    full-size layer (16 tokens, 512 experts, top-10) captured as one HIP graph
    and replayed; every replay's y equals the eager forward bit for bit, with
    other forwards (other routing, the same workspace) and synchronisations
    between the replays."""
    print_case("decode layer, graph replay vs eager")
    from block_scaled_fp4_nvfp4_amd.stack import LayerStack
    m = _lib()
    cfg, w13, w2 = decode_layer
    x = dev_bf16(synth.activations(cfg))
    ids, wts = synth.routing(cfg)
    layer = gpu_layer(cfg, w13, w2)
    n = 4
    st = LayerStack([layer] * n, [x] * n, [dev(ids)] * n, [dev(wts)] * n)
    st.eager()
    torch.cuda.synchronize()
    eager = host(st.ys[0]).copy()
    for y in st.ys[1:]:
        np.testing.assert_array_equal(host(y).view(np.uint32), eager.view(np.uint32))
    st.capture()
    ids2, wts2 = synth.routing(cfg.replace(input_seed=cfg.input_seed + 7))
    for rep in range(3):
        for y in st.ys:
            y.fill_(float("nan"))
        m.moe_forward(layer, x, dev(ids2), dev(wts2), st.workspace)  # other work in the shared workspace
        torch.cuda.synchronize()
        st.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(st.ys):
            np.testing.assert_array_equal(host(y).view(np.uint32), eager.view(np.uint32),
                                          err_msg=f"replay {rep}, forward {i}")


def test_many_tokens_uses_multipass_permutation(tiny):
    """1200 pairs (> 1024) go through the three-pass permutation."""
    print_case("tiny layer, 600 tokens")
    cfg, w13, w2, _, _, _ = tiny
    c = cfg.replace(tokens=600, input_seed=11)
    x = synth.activations(c)
    ids, wts = synth.routing(c)
    y, ws, lay = _run(gpu_layer(c, w13, w2), x, ids, wts)
    off, por, rop = moe.permute(ids, c.num_experts)
    np.testing.assert_array_equal(_ws_i32(ws, lay["offsets"], c.num_experts + 1), off)
    np.testing.assert_array_equal(_ws_i32(ws, lay["pair_of_row"], c.pairs), por)
    np.testing.assert_array_equal(_ws_i32(ws, lay["row_of_pair"], c.pairs), rop)
    y_ref = moe.moe_forward(OracleLayer(c, w13, w2).as_dict(), x, ids, wts)
    assert rel_fro(y, y_ref) < 1e-5


def test_decode_layer_mxfp4_x_mxfp8_gemv_path(decode_layer):
    """MXFP4 weights x dynamic MXFP8 activations at the decode shape (160
    pairs): the GEMVs on the exactly dequantized MXFP8 x and h; sampled tokens
    vs the oracle, and the quantized h bit-exact against the oracle's MXFP8
    of the GPU's own h."""
    print_case("decode layer, MXFP4 x MXFP8 GEMV path")
    cfg, w13, w2 = decode_layer
    c = cfg.replace(w_fmt="mxfp4", a_fmt="mxfp8")
    x = synth.activations(c)
    ids, wts = synth.routing(c)
    y, ws, lay = _run(gpu_layer(c, w13, w2), x, ids, wts)
    sample = [0, 9, 15]
    y_ref = moe.moe_forward(OracleLayer(c, w13, w2).as_dict(), x, ids, wts, sample_tokens=sample)
    err = rel_fro(y[sample], y_ref)
    print(f"relative Frobenius error {err:.3e}")
    assert err <= TOL
    from oracle import quant
    P, I = c.pairs, c.inter
    h = _ws_f32(ws, lay["h"], P * I).reshape(P, I)
    q = quant.quantize_mxfp8(h.astype(np.float64))
    codes = host(ws[lay["hq_codes"]:lay["hq_codes"] + P * I])
    np.testing.assert_array_equal(codes.reshape(P, I), q["codes"])


def test_decode_layer_fp8_block_tiled_weights_bit_identical(decode_layer):
    """16 tokens through a block-FP8 x FP8-row layer at the decode shape (the
    stack's retained layers): with tiled copies of W13 and W2 both grouped
    GEMMs read the same bytes in another order, so y is bit-identical to the
    row-major layer's; and within the layer bar of the oracle."""
    import block_scaled_fp4_nvfp4_amd as m
    print_case("decode layer, block FP8, tiled weights")
    cfg, w13, w2 = decode_layer
    c = cfg.replace(w_fmt="fp8_block", a_fmt="fp8_row", rule="rtn")
    x = synth.activations(c)
    ids, wts = synth.routing(c)
    layer = gpu_layer(c, w13, w2)
    y0, _, _ = _run(layer, x, ids, wts)
    layer.w13_tiled, _ = m.tile_weights(layer.w13, None, "fp8_block")
    layer.w2_tiled, _ = m.tile_weights(layer.w2, None, "fp8_block")
    y1, _, _ = _run(layer, x, ids, wts)
    np.testing.assert_array_equal(np.asarray(y0, np.float32).view(np.uint32),
                                  np.asarray(y1, np.float32).view(np.uint32))
    sample = [0, 15]
    y_ref = moe.moe_forward(OracleLayer(c, w13, w2).as_dict(), x, ids, wts, sample_tokens=sample)
    err = rel_fro(y1[sample], y_ref)
    print(f"relative Frobenius error {err:.3e}")
    assert err <= TOL
