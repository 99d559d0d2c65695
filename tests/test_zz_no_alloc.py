"""moe_fp4_forward_noalloc, the forward for callers that cannot allocate
(it takes its workspace from the library's per-device scratch array), against
moe_fp4_forward on the same inputs through the C ABI: y bit-identical (same
kernels in the same order), on two calls in a row where the second has fewer
tokens, for every path of the forward: the weight-only GEMVs, the MXFP4 x
MXFP8 decode GEMVs, the NVFP4 W4A4 grouped GEMMs with the shared expert, and
block FP8.  A problem larger than the scratch is refused before any launch."""
import numpy as np
import pytest

import synth

from gpu_util import dev, dev_bf16, gpu_ok, host, print_case, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def _pkg():
    import block_scaled_fp4_nvfp4_amd as m
    return m


def _device_layer(w_fmt, a_fmt, E, H, I, k, seed, shared_inter=0):
    """Weights N(0, 0.02) drawn on the device and quantized by the library."""
    m = _pkg()
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    w13 = (torch.randn(E, 2 * I, H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    rule = "4over6" if w_fmt in ("nvfp4", "mxfp4") else "rtn"
    q13, q2 = m.quantize(w13, w_fmt, rule), m.quantize(w2, w_fmt, rule)
    layer = m.MoELayer(w_fmt, a_fmt, E, H, I, k, q13["codes"], q13["scales"], q2["codes"], q2["scales"],
                       q13["tensor_scale"], q2["tensor_scale"])
    if shared_inter:
        s13 = (torch.randn(2 * shared_inter, H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        s2 = (torch.randn(H, shared_inter, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        a, b = m.quantize(s13, "mxfp8"), m.quantize(s2, "mxfp8")
        layer.shared_inter = shared_inter
        layer.ws13, layer.ws13_scale, layer.ws2, layer.ws2_scale = a["codes"], a["scales"], b["codes"], b["scales"]
        layer.shared_gate = (torch.randn(H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    torch.cuda.synchronize()
    return layer


def _inputs(T, E, H, k, seed):
    rs = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rs.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rs.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rs.random((T, k)).astype(np.float32) + 0.05
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    return dev_bf16(x), dev(ids), dev(w)


def _two_calls(layer, token_counts, seed):
    m = _pkg()
    E, H, k = layer.num_experts, layer.hidden, layer.top_k
    for i, T in enumerate(token_counts):
        print_case(f"noalloc {layer.w_fmt} x {layer.a_fmt}, E={E} H={H} I={layer.inter} k={k} "
                   f"shared={layer.shared_inter}, call {i + 1}: T={T}")
        x, ids, w = _inputs(T, E, H, k, seed + i)
        y_na = m.moe_forward_noalloc(layer, x, ids, w)
        ws = torch.zeros(m.workspace_size(layer, T), dtype=torch.uint8, device="cuda")
        y_ref = m.moe_forward(layer, x, ids, w, ws)
        torch.cuda.synchronize()
        a, b = host(y_na), host(y_ref)
        assert np.isfinite(a).all() and np.abs(a).max() > 0
        np.testing.assert_array_equal(a, b)


def test_noalloc_weight_only_gemv():
    _two_calls(_device_layer("nvfp4", "none", 64, 2560, 640, 10, 11), [16, 5], 100)


def test_noalloc_mxfp4_x_mxfp8_decode():
    _two_calls(_device_layer("mxfp4", "mxfp8", 64, 2560, 640, 10, 12), [16, 3], 200)


def test_noalloc_w4a4_grouped_with_shared_expert():
    _two_calls(_device_layer("nvfp4", "nvfp4", 8, 256, 128, 2, 13, shared_inter=128), [64, 16], 300)


def test_noalloc_block_fp8_grouped():
    _two_calls(_device_layer("fp8_block", "fp8_row", 16, 256, 256, 4, 14), [64, 20], 400)


def test_noalloc_refuses_more_than_its_scratch():
    m = _pkg()
    print_case("noalloc: workspace above the scratch maximum is refused")
    layer = _device_layer("nvfp4", "none", 64, 2560, 640, 10, 15)
    T = 8192
    assert m.workspace_size(layer, T) > m._lib.NOALLOC_SCRATCH_BYTES
    x, ids, w = _inputs(T, 64, 2560, 10, 500)
    y = torch.full((T, 2560), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(m.Fp4Error) as ei:
        m.moe_forward_noalloc(layer, x, ids, w, y)
    assert ei.value.status == -4
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing was launched
