"""Guard bands: every output buffer of fp4_quantize, moe_fp4_forward and
moe_fp4_tile_weights is surrounded by canary bytes that must read back
unchanged, and no input buffer changes.  The quantizer parks partial tensor
maxima inside code bytes (one-tensor path, chunked batches) and the NVFP4
gate_up GEMM leaves per-workgroup maxima in the workspace: an offset or size
mistake in any of them would land outside the buffers checked here."""
import ctypes

import numpy as np
import pytest

import synth
from oracle.formats import bf16_bits_from_f32

from gpu_util import dev, dev_bf16, gpu_layer, gpu_ok, host, print_case, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]

PAD = 4096
CANARY = 0xA5


def _pkg():
    import block_scaled_fp4_nvfp4_amd as m
    return m


class Guarded:
    """A device buffer of n bytes between two PAD-byte canary margins."""

    def __init__(self, n):
        self.n = n
        self.buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.uint8, device="cuda")

    @property
    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr() + PAD)

    def check(self, name):
        h = host(self.buf)
        bad_lo = np.nonzero(h[:PAD] != CANARY)[0]
        bad_hi = np.nonzero(h[PAD + self.n:] != CANARY)[0]
        assert bad_lo.size == 0, f"{name}: {bad_lo.size} bytes written below the buffer (first at -{PAD - bad_lo[0]})"
        assert bad_hi.size == 0, f"{name}: {bad_hi.size} bytes written past the buffer (first at +{bad_hi[0]})"

    def inner(self):
        return self.buf[PAD:PAD + self.n]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


SCALE_BYTES = {"nvfp4": lambda c: c // 16, "mxfp4": lambda c: c // 32, "mxfp8": lambda c: c // 32,
               "fp8_row": lambda c: c // 128 * 4}


@pytest.mark.parametrize("fmt,rule,B,R,C", [
    ("nvfp4", "4over6", 1, 512, 1024),     # one tensor: maxima parked in its own code bytes
    ("nvfp4", "sweep", 3, 256, 512),
    ("nvfp4", "4over6", 19, 1024, 1024),   # chunked batch: next chunk's maxima in its code bytes
    ("mxfp4", "4over6", 2, 128, 512),
    ("mxfp8", "rtn", 2, 128, 512),
    ("fp8_row", "rtn", 2, 128, 512),
    ("fp8_block", "rtn", 2, 256, 384),
])
def test_quantize_writes_stay_in_their_buffers(fmt, rule, B, R, C):
    print_case(f"guard: fp4_quantize {fmt}/{rule} {B}x{R}x{C}")
    m = _pkg()
    L = m.lib()
    rng = np.random.default_rng(B * 7 + R)
    x = rng.standard_normal((B, R, C), dtype=np.float32) * np.float32(0.02)
    bits = bf16_bits_from_f32(x)
    xd = dev_bf16(bits)
    before = host(xd).copy()
    fp4 = fmt in ("nvfp4", "mxfp4")
    codes = Guarded(B * R * C // (2 if fp4 else 1))
    sb = B * (R // 128) * (C // 128) * 4 if fmt == "fp8_block" else B * R * SCALE_BYTES[fmt](C)
    scales = Guarded(sb)
    ts = Guarded(4 * B)
    m4 = Guarded(B * R * C // (16 if fmt == "nvfp4" else 32)) if fp4 else None
    st = L.fp4_quantize(m.FMT[fmt], m.RULE[rule], 0, ctypes.c_void_p(xd.data_ptr()), 0, B, R, C, codes.ptr,
                        scales.ptr, ts.ptr if fmt == "nvfp4" else None, m4.ptr if m4 else None, _stream())
    assert st == 0, L.fp4_last_error()
    torch.cuda.synchronize()
    for name, g in (("codes", codes), ("scales", scales), ("tensor_scale", ts), ("m4", m4)):
        if g is not None:
            g.check(name)
    np.testing.assert_array_equal(host(xd), before)
    # and the guarded outputs equal an unguarded call's
    q = m.quantize(xd, fmt, rule, want_m4=fp4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(codes.inner()), host(q["codes"]).reshape(-1))
    if fmt == "nvfp4":
        np.testing.assert_array_equal(host(ts.inner()).view(np.float32), host(q["tensor_scale"]))


def _tiny(a_fmt, w_fmt="nvfp4", tokens=64, shared=False, rule="4over6"):
    cfg = synth.CONFIGS["tiny"].replace(a_fmt=a_fmt, w_fmt=w_fmt, tokens=tokens, input_seed=5, rule=rule)
    if shared:
        cfg = cfg.replace(shared_inter=128)
    w13, w2 = synth.layer_weights(cfg)
    sh = synth.shared_expert(cfg) if shared else None
    return cfg, gpu_layer(cfg, w13, w2, shared=sh)


@pytest.mark.parametrize("w_fmt,a_fmt,tokens,shared", [
    ("nvfp4", "none", 64, False),
    ("nvfp4", "nvfp4", 64, True),
    ("nvfp4", "nvfp4", 600, False),    # three-pass permutation, gate_up maxima for S_h
    ("mxfp4", "mxfp8", 32, False),     # decode GEMVs on dequantized MXFP8
    ("mxfp4", "mxfp8", 600, False),    # grouped MX GEMMs, MXFP8 h from the gate_up epilogue
    ("fp8_block", "fp8_row", 600, False),
])
def test_forward_writes_stay_in_their_buffers(w_fmt, a_fmt, tokens, shared):
    print_case(f"guard: moe_fp4_forward {w_fmt} x {a_fmt}, {tokens} tokens, shared={shared}")
    m = _pkg()
    L = m.lib()
    cfg, layer = _tiny(a_fmt, w_fmt, tokens, shared, rule="rtn" if w_fmt == "fp8_block" else "4over6")
    x = dev_bf16(synth.activations(cfg))
    ids_np, wts_np = synth.routing(cfg)
    ids, wts = dev(ids_np), dev(wts_np)
    inputs = {n: (t, host(t).copy()) for n, t in
              (("x", x), ("ids", ids), ("weights", wts), ("w13", layer.w13), ("w13_scale", layer.w13_scale),
               ("w2", layer.w2), ("w2_scale", layer.w2_scale))}
    T, H = cfg.tokens, cfg.hidden
    wsz = m.workspace_size(layer, T)
    ws = Guarded(wsz)
    y = Guarded(T * H * 4)
    s = layer.struct()
    st = L.moe_fp4_forward(ctypes.byref(s), ctypes.c_void_p(x.data_ptr()), T, ctypes.c_void_p(ids.data_ptr()),
                           ctypes.c_void_p(wts.data_ptr()), y.ptr, ws.ptr, wsz, _stream())
    assert st == 0, L.fp4_last_error()
    torch.cuda.synchronize()
    ws.check("workspace")
    y.check("y")
    for n, (t, h) in inputs.items():
        np.testing.assert_array_equal(host(t), h, err_msg=f"input {n} changed")
    ref = m.moe_forward(layer, x, ids, wts)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y.inner()).view(np.float32).reshape(T, H), host(ref))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "fp8_block"])
def test_tile_weights_writes_stay_in_their_buffers(fmt):
    print_case(f"guard: moe_fp4_tile_weights {fmt}")
    m = _pkg()
    L = m.lib()
    E, R, C = 3, 128, 512
    rng = np.random.default_rng(9)
    bits = bf16_bits_from_f32(rng.standard_normal((E, R, C), dtype=np.float32) * np.float32(0.02))
    q = m.quantize(dev_bf16(bits), fmt, "rtn")
    torch.cuda.synchronize()
    codes_before = host(q["codes"]).copy()
    scales_before = host(q["scales"]).copy()
    fp4 = fmt != "fp8_block"
    tc = Guarded(q["codes"].numel())
    tsc = Guarded(q["scales"].numel()) if fp4 else None
    st = L.moe_fp4_tile_weights(m.FMT[fmt], ctypes.c_void_p(q["codes"].data_ptr()),
                                ctypes.c_void_p(q["scales"].data_ptr()) if fp4 else None, E, R, C, tc.ptr,
                                tsc.ptr if fp4 else None, _stream())
    assert st == 0, L.fp4_last_error()
    torch.cuda.synchronize()
    tc.check("tiled codes")
    if tsc:
        tsc.check("tiled scales")
    np.testing.assert_array_equal(host(q["codes"]), codes_before)
    np.testing.assert_array_equal(host(q["scales"]), scales_before)
    # the same bytes, rearranged
    assert sorted(host(tc.inner()).tolist()) == sorted(codes_before.reshape(-1).tolist())
