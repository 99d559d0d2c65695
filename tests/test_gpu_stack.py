"""The mixed-precision routed-expert stack (MXFP4-FP8-R12 card, "Quantization
format" and "Retained layers": listed layers keep block-FP8 experts with
dynamic FP8 activations, the rest run MXFP4 x dynamic MXFP8) run eagerly and
as one captured HIP graph (the card's decode graphs).

Bar: every layer's y within 2e-3 relative Frobenius of the oracle (the layer's
bar; the MXFP8 / FP8 requantization of h puts these modes near 2e-4); graph
replays bit-identical to the eager pass, replayed several times with other
GPU work and synchronisations in between."""
import numpy as np
import pytest

import synth
from oracle import moe

from gpu_util import OracleLayer, dev, dev_bf16, gpu_layer, gpu_ok, host, print_case, rel_fro, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def _small_stack():
    cfgs = synth.stack_configs(n_layers=4, tokens=64, num_experts=8, top_k=2, hidden=256, inter=128,
                               fp8_layers=(1, 3))
    from block_scaled_fp4_nvfp4_amd.stack import LayerStack
    layers, xs, ids, ws, refs = [], [], [], [], []
    for cfg in cfgs:
        w13, w2 = synth.layer_weights(cfg)
        x = synth.activations(cfg)
        i, w = synth.routing(cfg)
        layers.append(gpu_layer(cfg, w13, w2))
        xs.append(dev_bf16(x))
        ids.append(dev(i))
        ws.append(dev(w))
        refs.append(moe.moe_forward(OracleLayer(cfg, w13, w2).as_dict(), x, i, w))
    return cfgs, LayerStack(layers, xs, ids, ws), refs


def test_mixed_stack_eager_and_graph():
    print_case("4-layer mixed MXFP4 / block-FP8 stack, eager then graph")
    cfgs, st, refs = _small_stack()
    assert [c.w_fmt for c in cfgs] == ["mxfp4", "fp8_block", "mxfp4", "fp8_block"]
    st.eager()
    torch.cuda.synchronize()
    eager = [host(y).copy() for y in st.ys]
    for l, (y, ref) in enumerate(zip(eager, refs)):
        err = rel_fro(y, ref)
        print(f"layer {l} ({cfgs[l].w_fmt}): relative Frobenius error {err:.3e}")
        assert err <= 2e-3, f"layer {l} ({cfgs[l].w_fmt})"
    st.capture()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        for y in st.ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        st.replay()
        torch.cuda.synchronize()
        for l, y in enumerate(st.ys):
            np.testing.assert_array_equal(host(y).view(np.uint32), eager[l].view(np.uint32),
                                          err_msg=f"replay {rep}, layer {l}")
        scratch.normal_()      # other work on the stream between replays
        torch.cuda.synchronize()


def test_graph_capture_with_the_shared_expert_stream():
    """A W4A4 layer with the MXFP8 shared expert, whose launches fork onto the
    library's helper stream and join back: captured as one graph, every replay
    equals the eager pass bit for bit, and the eager pass matches the oracle."""
    print_case("graph capture of a layer with the shared expert")
    from block_scaled_fp4_nvfp4_amd.stack import LayerStack
    cfg = synth.CONFIGS["tiny"].replace(a_fmt="nvfp4", shared_inter=128)
    w13, w2 = synth.layer_weights(cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    shared = synth.shared_expert(cfg)
    st = LayerStack([gpu_layer(cfg, w13, w2, shared=shared)], [dev_bf16(x)], [dev(ids)], [dev(wts)])
    st.eager()
    torch.cuda.synchronize()
    eager = host(st.ys[0]).copy()
    ref = moe.moe_forward(OracleLayer(cfg, w13, w2, shared=shared).as_dict(), x, ids, wts)
    assert rel_fro(eager, ref) <= 2e-3
    st.capture()
    for rep in range(3):
        st.ys[0].fill_(float("nan"))
        torch.cuda.synchronize()
        st.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(st.ys[0]).view(np.uint32), eager.view(np.uint32),
                                      err_msg=f"replay {rep}")
