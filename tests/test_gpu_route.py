"""GPU top-k routing (moe_fp4_route) against the oracle's routing, and the
routing width and shared-expert width as runtime values (FP4-Local-AZ card,
"What is different from NVIDIA's checkpoint": 10 or 5 routed experts, a
640-wide shared expert zero-padded to 1280 with output unchanged).

Bar: expert ids exact (the selection compares the same fp32 values on both
sides); weights within one fp32 ulp (both compute the softmax in fp64 and
round once; their exp and summation orders differ in the last fp64 bits)."""
import numpy as np
import pytest

import synth
from oracle import moe

from gpu_util import OracleLayer, dev, dev_bf16, gpu_layer, gpu_ok, host, print_case, rel_fro, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def _lib():
    import block_scaled_fp4_nvfp4_amd as m
    return m


def _route(lg, bias, k):
    ids, w = _lib().route(dev(np.ascontiguousarray(lg, np.float32)), k,
                          None if bias is None else dev(np.asarray(bias, np.float32)))
    torch.cuda.synchronize()
    return host(ids), host(w)


def _check(lg, bias, k):
    ids, w = _route(lg, bias, k)
    o_ids, o_w = moe.route(lg, bias, k)
    np.testing.assert_array_equal(ids, o_ids)
    np.testing.assert_array_max_ulp(w, o_w, maxulp=1)
    return ids, w


@pytest.mark.parametrize("name", ["decode", "prefill_nvfp4", "prefill_mxfp4"])
def test_route_workload_shapes(name):
    cfg = synth.CONFIGS[name]
    print_case(f"route {name}: T={cfg.tokens} E={cfg.num_experts} k={cfg.top_k}")
    lg, b = synth.router_logits(cfg), synth.router_bias(cfg)
    ids, w = _check(lg, b if cfg.router_bias else None, cfg.top_k)
    # the layer's own input generator routes identically
    s_ids, _ = synth.routing(cfg)
    np.testing.assert_array_equal(ids, s_ids)


@pytest.mark.parametrize("E,k", [(8, 2), (100, 7), (64, 1), (32, 32), (1024, 10), (512, 5)])
def test_route_edge_widths_and_ties(E, k):
    print_case(f"route E={E} k={k}")
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.standard_normal((37, E)).astype(np.float32)
    _check(lg, None, k)
    # heavy ties: values on a coarse grid, equal values resolved by expert id
    tied = (np.round(lg * 2) / 2).astype(np.float32)
    _check(tied, None, k)
    _check(np.zeros((5, E), np.float32), None, k)
    bias = rng.standard_normal(E).astype(np.float32)
    _check(lg, bias, k)


def test_route_runtime_k_prefix():
    """k = 5 and k = 10 on the same logits: the first five ids agree."""
    print_case("route runtime k")
    cfg = synth.CONFIGS["decode"]
    lg = synth.router_logits(cfg)
    ids10, w10 = _route(lg, None, 10)
    ids5, w5 = _route(lg, None, 5)
    np.testing.assert_array_equal(ids5, ids10[:, :5])
    assert np.all(w5 >= w10[:, :5])


def test_gpu_routing_drives_the_decode_layer():
    """Routing on the GPU, then the layer with k = 10 and, from the same
    weights and library, k = 5 (the runtime routing width), against the oracle."""
    cfg = synth.CONFIGS["decode"]
    w13, w2 = synth.layer_weights(cfg)
    x = synth.activations(cfg)
    lg = synth.router_logits(cfg)
    m = _lib()
    layer = gpu_layer(cfg, w13, w2)
    ol = OracleLayer(cfg, w13, w2).as_dict()
    for k in (10, 5):
        print_case(f"decode layer routed on the GPU, k={k}")
        ids_d, w_d = m.route(dev(lg), k)
        layer.top_k = k
        ws = torch.zeros(m.workspace_size(layer, cfg.tokens), dtype=torch.uint8, device="cuda")
        y = host(m.moe_forward(layer, dev_bf16(x), ids_d, w_d, ws))
        ids, wts = host(ids_d), host(w_d)
        sample = [1, 8, 14]
        y_ref = moe.moe_forward(ol, x, ids, wts, sample_tokens=sample)
        assert rel_fro(y[sample], y_ref) < 1e-5


def test_shared_expert_zero_padded_width_is_bit_identical():
    """A shared expert of width 128 and the same expert zero-padded to 256
    (extra gate/up rows and down columns zero) give the same y bit for bit."""
    print_case("shared expert zero padding")
    m = _lib()
    cfg = synth.CONFIGS["tiny"].replace(shared_inter=128)
    w13, w2 = synth.layer_weights(cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    s13, s2, g = synth.shared_expert(cfg)
    S, H = cfg.shared_inter, cfg.hidden
    z13 = np.zeros((S, H), np.uint16)
    s13p = np.concatenate([s13[:S], z13, s13[S:], z13], axis=0)
    s2p = np.concatenate([s2, np.zeros((H, S), np.uint16)], axis=1)
    ys = []
    for shared in ((s13, s2, g), (s13p, s2p, g)):
        layer = gpu_layer(cfg, w13, w2, shared=shared)
        ws = torch.zeros(m.workspace_size(layer, cfg.tokens), dtype=torch.uint8, device="cuda")
        ys.append(host(m.moe_forward(layer, dev_bf16(x), dev(ids), dev(wts), ws)))
    np.testing.assert_array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
