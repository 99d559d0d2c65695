"""GPU parity of fp4_quantize_hessian (the Hessian-weighted NVFP4 scale
search; Local-Hessian NVFP4 card, "What is different about it" and
"Results") against oracle/quant.py::quantize_nvfp4_hessian: codes, scales,
tensor scales and chosen offsets bit-exact, on random experts with synthetic
calibration covariances (thin experts included), f32 inputs, H = I (which
must equal the GPU's own scale sweep), the hand-worked near-tie blocks of
tests/golden/hessian_worked_example.txt, and one expert of each model shape.
Bytes around the outputs stay untouched."""
import numpy as np
import pytest

import synth
from oracle import quant as Q
from oracle.formats import bf16_bits_from_f32, bf16_to_f64, pack_nibbles

from gpu_util import dev, dev_bf16, gpu_ok, host, print_case, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def _pkg():
    import block_scaled_fp4_nvfp4_amd as m
    return m


def _bf16_bits(rng, shape, std=0.02, heavy=False):
    v = rng.standard_t(4, shape) if heavy else rng.standard_normal(shape)
    return bf16_bits_from_f32((v * std).astype(np.float32))


def _check(x_f64, H, n_rows, q_gpu, e, tag):
    ref = Q.quantize_nvfp4_hessian(x_f64, H, int(n_rows))
    codes = host(q_gpu["codes"][e])
    np.testing.assert_array_equal(codes, pack_nibbles(ref["codes"]), err_msg=f"{tag}: codes")
    np.testing.assert_array_equal(host(q_gpu["scales"][e]), ref["scales"], err_msg=f"{tag}: scales")
    assert host(q_gpu["tensor_scale"])[e] == ref["tensor_scale"], f"{tag}: tensor scale"
    if q_gpu["choice"] is not None:
        np.testing.assert_array_equal(host(q_gpu["choice"][e]), ref["choice"], err_msg=f"{tag}: choice")
    return ref


def test_hessian_random_experts_bf16_and_thin_rule():
    print_case("hessian: 4 experts 64 x 256 bf16, calibration rows [200, 0, 30, 64]")
    m = _pkg()
    rng = np.random.default_rng(1)
    E, R, C = 4, 64, 256
    bits = np.stack([_bf16_bits(rng, (R, C), heavy=e % 2 == 1) for e in range(E)])
    n = np.array([200, 0, 30, 64], np.int32)
    H = np.stack([synth.calibration_hessian(3, e, C, max(int(n[e]), 1)) for e in range(E)])
    q = m.quantize_hessian(dev_bf16(bits), dev(H), dev(n), want_choice=True)
    torch.cuda.synchronize()
    moved = 0
    for e in range(E):
        ref = _check(bf16_to_f64(bits[e]), H[e], n[e], q, e, f"expert {e}")
        moved += int((ref["choice"] > 0).sum())
        if n[e] < 64:
            assert not ref["choice"].any()
    assert moved > 0


def test_hessian_f32_inputs():
    print_case("hessian: f32 inputs, 2 experts 32 x 128")
    m = _pkg()
    rng = np.random.default_rng(2)
    x = (rng.standard_t(4, (2, 32, 128)) * 0.02).astype(np.float32)
    n = np.array([500, 100], np.int32)
    H = np.stack([synth.calibration_hessian(4, e, 128, int(n[e])) for e in range(2)])
    q = m.quantize_hessian(dev(x), dev(H), dev(n), want_choice=True)
    torch.cuda.synchronize()
    for e in range(2):
        _check(x[e].astype(np.float64), H[e], n[e], q, e, f"f32 expert {e}")


def test_hessian_identity_equals_the_gpu_sweep():
    print_case("hessian: H = I equals FP4_RULE_SWEEP on the GPU")
    m = _pkg()
    rng = np.random.default_rng(3)
    bits = _bf16_bits(rng, (3, 128, 512), heavy=True)
    H = np.broadcast_to(np.eye(16, dtype=np.float32), (3, 32, 16, 16)).copy()
    x = dev_bf16(bits)
    q = m.quantize_hessian(x, dev(H), dev(np.full(3, 64, np.int32)), want_choice=True)
    s = m.quantize(x, "nvfp4", "sweep", want_m4=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q["codes"]), host(s["codes"]))
    np.testing.assert_array_equal(host(q["scales"]), host(s["scales"]))
    np.testing.assert_array_equal(host(q["choice"]), host(s["m4"]))
    np.testing.assert_array_equal(host(q["tensor_scale"]), host(s["tensor_scale"]))


def _near_tie_expert():
    """Rows of the hand-worked blocks A-D (columns 0-63) in several scalings
    and near-tie variants of block D, plus 2688 in the last row so that the
    tensor scale amax/2688 is exactly 1."""
    x = np.zeros((40, 64), np.float32)
    x[0, 0:2] = [6, 5]
    x[0, 16:18] = [6, -5]
    x[0, 32:34] = [6, 5]
    x[0, 48:51] = [6, 6, 0.3125]
    rng = np.random.default_rng(4)
    for r in range(1, 39):
        for b in range(4):
            a = float(rng.choice([4.5, 5.0, 5.5, 6.0, 7.0]))
            x[r, 16 * b] = a
            x[r, 16 * b + 1] = a if b == 3 else float(rng.choice([-5.0, 3.0, 4.5, 5.0]))
            x[r, 16 * b + 2] = float(np.float32(rng.uniform(0.05, 0.9)))
    x[39, 60] = 2688.0
    bits = bf16_bits_from_f32(x)
    H = np.stack([np.eye(16) for _ in range(4)])
    H[0, 0, 1] = H[0, 1, 0] = 0.9
    H[1, 0, 1] = H[1, 1, 0] = -0.9
    H[2] = 0.0
    H[2, 0, 0] = 1.0
    H[3] = 0.0
    H[3, :2, :2] = [[1.0, -1.0], [-1.0, 1.0]]
    H[3, 2, 2] = 2.0 ** -50
    return bits, H.astype(np.float32)


def test_hessian_hand_worked_and_near_tie_blocks():
    print_case("hessian: hand-worked blocks and near ties (exact path)")
    m = _pkg()
    bits, H = _near_tie_expert()
    q = m.quantize_hessian(dev_bf16(bits[None]), dev(H[None]), dev(np.array([64], np.int32)), want_choice=True)
    torch.cuda.synchronize()
    assert host(q["tensor_scale"])[0] == 1.0
    ref = _check(bf16_to_f64(bits), H, 64, q, 0, "near ties")
    # the fixture's answers on row 0
    np.testing.assert_array_equal(ref["scales"][0], [0x3B, 0x3B, 0x38, 0x38])


@pytest.mark.parametrize("shape,n", [((1280, 2560), 5007), ((2560, 640), 812)])
def test_hessian_full_size_expert(shape, n):
    """One expert matrix of each model shape (fused gate_up 1280 x 2560 with
    the hidden-size Hessian, down 2560 x 640 with the intermediate-size one)."""
    print_case(f"hessian: full-size expert {shape}, {n} calibration rows")
    m = _pkg()
    rng = np.random.default_rng(5)
    bits = _bf16_bits(rng, shape, heavy=True)
    H = synth.calibration_hessian(6, 0, shape[1], n)
    q = m.quantize_hessian(dev_bf16(bits[None]), dev(H[None]), dev(np.array([n], np.int32)), want_choice=True)
    torch.cuda.synchronize()
    _check(bf16_to_f64(bits), H, n, q, 0, f"full size {shape}")


def test_hessian_writes_stay_in_their_buffers():
    print_case("hessian: canary bytes around codes, scales, tensor scales and choices")
    m = _pkg()
    rng = np.random.default_rng(7)
    E, R, C = 3, 48, 128
    bits = _bf16_bits(rng, (E, R, C))
    H = np.stack([synth.calibration_hessian(8, e, C, 100) for e in range(E)])
    pad = 256
    lib = m.lib()
    import ctypes

    def guarded(n):
        return torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")

    nc, ns = E * R * C // 2, E * R * C // 16
    codes, scales, choice, ts = guarded(nc), guarded(ns), guarded(ns), guarded(4 * E)
    x, h, rows = dev_bf16(bits), dev(H), dev(np.full(E, 100, np.int32))  # kept alive past the launch
    vp = ctypes.c_void_p
    m._lib._check(lib.fp4_quantize_hessian(
        vp(x.data_ptr()), 0, E, R, C, vp(h.data_ptr()), vp(rows.data_ptr()),
        vp(codes.data_ptr() + pad), vp(scales.data_ptr() + pad), vp(ts.data_ptr() + pad),
        vp(choice.data_ptr() + pad), vp(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()
    for name, buf, n in (("codes", codes, nc), ("scales", scales, ns), ("choice", choice, ns),
                         ("tensor_scale", ts, 4 * E)):
        hb = host(buf)
        assert np.all(hb[:pad] == 0xA5) and np.all(hb[pad + n:] == 0xA5), name
    # and the guarded outputs are the oracle's
    ref = Q.quantize_nvfp4_hessian(bf16_to_f64(bits[1]), H[1], 100)
    np.testing.assert_array_equal(host(scales)[pad + ns // E:pad + 2 * ns // E].reshape(R, C // 16), ref["scales"])
