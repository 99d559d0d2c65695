"""GPU quantizer / dequantizer parity through the C ABI: codes and scales are
bit-exact against the oracle (all three scale rules: RTN, 4/6 and the
scale sweep); dequantized values equal the oracle's exact values rounded once
to f32 (bf16: then rounded to bf16)."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import quant as Q

from gpu_util import dev, dev_bf16, gpu_ok, host, print_case, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")]


def _lib():
    import block_scaled_fp4_nvfp4_amd as m
    return m


def _oracle_q(fmt, x64, rule):
    if fmt == "nvfp4":
        return Q.quantize_nvfp4(x64, rule)
    if fmt == "mxfp4":
        return Q.quantize_mxfp4(x64, rule)
    if fmt == "mxfp8":
        return Q.quantize_mxfp8(x64)
    if fmt == "fp8_row":
        return Q.quantize_fp8_rows(x64)
    if fmt == "fp8_block":
        return Q.quantize_fp8_block_weight(x64)
    raise ValueError(fmt)


def _compare(fmt, rule, xt, x64_per_tensor):
    """Quantize xt ([B, R, C] device) on the GPU and compare every tensor."""
    m = _lib()
    q = m.quantize(xt, fmt, rule, want_m4=fmt in ("nvfp4", "mxfp4"))
    torch.cuda.synchronize()
    codes, scales = host(q["codes"]), host(q["scales"])
    for b, x64 in enumerate(x64_per_tensor):
        o = _oracle_q(fmt, x64, rule)
        oc = F.pack_nibbles(o["codes"]) if fmt in ("nvfp4", "mxfp4") else o["codes"]
        np.testing.assert_array_equal(codes[b], oc, err_msg=f"{fmt}/{rule} codes, tensor {b}")
        if fmt in ("fp8_row", "fp8_block"):
            np.testing.assert_array_equal(scales[b].view(np.uint32), o["scales"].view(np.uint32))
        else:
            np.testing.assert_array_equal(scales[b], o["scales"], err_msg=f"{fmt}/{rule} scales, tensor {b}")
        if fmt == "nvfp4":
            assert host(q["tensor_scale"])[b].view(np.uint32) == np.float32(o["tensor_scale"]).view(np.uint32)
        if q["m4"] is not None:
            np.testing.assert_array_equal(host(q["m4"])[b].astype(bool), o["m4"])
            if "choice" in o:  # NVFP4 sweep: offset of the chosen scale code
                np.testing.assert_array_equal(host(q["m4"])[b], o["choice"], err_msg=f"{fmt}/{rule} choice, tensor {b}")
    return q


@pytest.mark.parametrize("fmt,rule", [("nvfp4", "4over6"), ("nvfp4", "rtn"), ("nvfp4", "sweep"),
                                      ("mxfp4", "4over6"), ("mxfp4", "rtn"), ("mxfp4", "sweep")])
def test_fp4_weights_bit_exact_tiny_layer(fmt, rule):
    print_case(f"tiny layer weights {fmt}/{rule}")
    cfg = synth.CONFIGS["tiny"]
    w13, w2 = synth.layer_weights(cfg)
    for w in (w13, w2):
        _compare(fmt, rule, dev_bf16(w), [F.bf16_to_f64(w[e]) for e in range(w.shape[0])])


def test_fp4_adversarial_blocks_bit_exact():
    print_case("adversarial blocks")
    rows = [
        [2688, 112, 336, 560, 784, 1120, 1568, 2240, -224, -0.0, 100, 120, 448, 672, 896, 1344] * 2,
        [0.0] * 32, [-0.0] * 32,
        [2688 * 2.0 ** -14] + [0.0] * 31,
        [2688 * 2.0 ** -20] * 32,
        [1792.0, -1792.0] * 16,
        [6.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.0] * 4,
        [8, 4, 2, 6, 1, 3, 0, -8, -4, -2, -6, -1, -3, -0.0, 8, 4] * 2,
    ]
    x = np.array(rows, np.float32)
    # add E2M1 tie points at many scales
    rng = np.random.default_rng(0)
    ties = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32)[None, :]
            * np.exp2(rng.integers(-8, 8, (24, 1))).astype(np.float32))
    x = np.concatenate([x, ties])
    bits = F.bf16_bits_from_f32(x)
    x64 = F.bf16_to_f64(bits)
    for fmt in ("nvfp4", "mxfp4"):
        for rule in ("4over6", "rtn", "sweep"):
            _compare(fmt, rule, dev_bf16(bits)[None], [x64])


def _structured_near_tie_tensors():
    """Tensors whose NVFP4 thresholds m*s*S land within S's rounding error of
    bf16 inputs: S = amax/2688 with 2688 = 21 * 2^7, and m*s = 21 * 2^j for
    (m, s) = (3.5, 6*2^j), (1.75, 12*2^j), (0.75, 28*2^j), so values a*2^-k that
    share the tensor amax a's significand sit next to a threshold."""
    amaxes = [1.0078125, 1.5234375, 1.2421875, 1.9921875, 1.3359375, 1.6640625]
    tensors = []
    for a in amaxes:
        rows = [[a] + [a * 2.0 ** -k for k in range(1, 16)]]
        for t in range(0, 8):  # block max a*2^-t: s6 = 448*2^-t (m = 0.75 ties)
            rows.append([(-1) ** k * a * 2.0 ** -(t + k % 9) for k in range(16)])
        for s_target in (6.0, 12.0, 24.0, 3.0):  # block max giving s6 = s_target
            bmax = a * 6.0 * s_target / 2688.0
            rows.append([bmax] + [(-1) ** k * a * 2.0 ** -(5 + k % 8) for k in range(15)])
        rows.append([0.0] * 16)
        tensors.append(np.array(rows, np.float32).reshape(-1, 32))
    x = np.stack(tensors)
    return F.bf16_bits_from_f32(x)


def test_fp4_structured_near_ties_bit_exact():
    print_case("structured near-ties of NVFP4 thresholds")
    bits = _structured_near_tie_tensors()
    x64 = [F.bf16_to_f64(bits[b]) for b in range(bits.shape[0])]
    for rule in ("4over6", "rtn", "sweep"):
        _compare("nvfp4", rule, dev_bf16(bits), x64)
    # the f32 path meets the same thresholds
    xf = F.bf16_to_f64(bits).astype(np.float32)
    for rule in ("4over6", "sweep"):
        _compare("nvfp4", rule, dev(xf), [xf[b].astype(np.float64) for b in range(xf.shape[0])])


def test_fp4_f32_inputs_bit_exact():
    print_case("f32 inputs")
    rng = np.random.default_rng(1)
    x = (rng.standard_t(3, (3, 64, 256)) * 0.03).astype(np.float32)
    x[0, 0, :16] = np.float32(1e-40)  # subnormal block
    for fmt in ("nvfp4", "mxfp4"):
        for rule in ("4over6", "rtn", "sweep"):
            _compare(fmt, rule, dev(x), [x[b].astype(np.float64) for b in range(3)])


@pytest.mark.parametrize("fmt", ["mxfp8", "fp8_row", "fp8_block"])
def test_fp8_formats_bit_exact(fmt):
    print_case(f"fp8 format {fmt}")
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 256, 512)).astype(np.float32) * np.exp2(
        rng.integers(-6, 6, (2, 256, 1))).astype(np.float32)
    x[0, :128, :128] = 0.0
    bits = F.bf16_bits_from_f32(x)
    _compare(fmt, "rtn", dev_bf16(bits), [F.bf16_to_f64(bits[b]) for b in range(2)])
    _compare(fmt, "rtn", dev(x), [x[b].astype(np.float64) for b in range(2)])


def _e4m3_midpoint_rows():
    """Rows of 128 values that put E4M3 quotients exactly on midpoints (normal
    and subnormal, both parities) and one float step either side of them.
    Each row's max is 448 * 1.25 (an FP8 row scale of exactly 1.25; an MXFP8
    block exponent of 1 for its first 32 values), so every quotient is exact."""
    grid = np.array(sorted(set(F.E4M3_GRID.tolist())), np.float64)
    grid = grid[np.isfinite(grid) & (grid >= 0) & (grid <= 448)]
    mids = (grid[:-1] + grid[1:]) / 2
    rows = []
    for sub in (mids[mids < 2.0 ** -6], mids[(mids >= 2.0 ** -6) & (mids < 2.0)], mids[mids >= 2.0]):
        for lo in range(0, len(sub), 42):
            part = sub[lo:lo + 42] * 1.25
            a = np.concatenate([part, np.nextafter(part.astype(np.float32), np.float32(np.inf)),
                                np.nextafter(part.astype(np.float32), np.float32(0))]).astype(np.float32)
            row = np.zeros(128, np.float32)
            row[0] = 448 * 1.25
            row[1:1 + len(a)] = a[:127]
            row[1::2] *= -1
            rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("fmt", ["mxfp8", "fp8_row"])
def test_fp8_midpoints_and_subnormals_bit_exact(fmt):
    """The E4M3 codes come from the hardware convert: exact ties (even code),
    subnormal codes and one-ulp neighbours of ties against exact rounding."""
    print_case(f"e4m3 midpoints {fmt}")
    x = _e4m3_midpoint_rows()[None]
    _compare(fmt, "rtn", dev(x), [x[0].astype(np.float64)])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "mxfp8", "fp8_row", "fp8_block"])
def test_dequantize_is_the_rounded_exact_value(fmt):
    print_case(f"dequantize {fmt}")
    m = _lib()
    rng = np.random.default_rng(3)
    x = (rng.standard_t(4, (2, 128, 256)) * 0.02).astype(np.float32)
    bits = F.bf16_bits_from_f32(x)
    xt = dev_bf16(bits)
    q = m.quantize(xt, fmt, "4over6")
    f32 = host(m.dequantize(q, fmt, xt.shape, torch.float32))
    b16 = host(m.dequantize(q, fmt, xt.shape, torch.bfloat16))
    codes, scales = host(q["codes"]), host(q["scales"])
    for b in range(2):
        if fmt == "nvfp4":
            exact = Q.dequantize_nvfp4(F.unpack_nibbles(codes[b]), scales[b], host(q["tensor_scale"])[b])
        elif fmt == "mxfp4":
            exact = Q.dequantize_mxfp4(F.unpack_nibbles(codes[b]), scales[b])
        elif fmt == "mxfp8":
            exact = Q.dequantize_mxfp8(codes[b], scales[b])
        elif fmt == "fp8_row":
            exact = Q.dequantize_fp8_rows(codes[b], scales[b])
        else:
            exact = Q.dequantize_fp8_block_weight(codes[b], scales[b])
        want32 = exact.astype(np.float32)
        np.testing.assert_array_equal(f32[b].view(np.uint32), want32.view(np.uint32))
        np.testing.assert_array_equal(b16[b], F.bf16_bits_from_f32(want32))


def test_decode_layer_sampled_experts_and_determinism():
    """Two experts of the 512-expert layer at its real shapes, and a repeat run
    giving identical bytes (two machines building byte-identical trees, QAD5500
    card, "Verification")."""
    print_case("decode-shape experts")
    m = _lib()
    cfg = synth.CONFIGS["decode"]
    ids = [0, 311]
    w13, w2 = synth.layer_weights(cfg, experts=ids)
    t13 = dev_bf16(w13)
    q1 = _compare("nvfp4", "4over6", t13, [F.bf16_to_f64(w13[i]) for i in range(2)])
    q2 = m.quantize(t13, "nvfp4", "4over6")
    torch.cuda.synchronize()
    assert torch.equal(q1["codes"], q2["codes"]) and torch.equal(q1["scales"], q2["scales"])
    _compare("nvfp4", "4over6", dev_bf16(w2), [F.bf16_to_f64(w2[i]) for i in range(2)])


def test_static_tensor_scale_and_error_codes():
    print_case("static tensor scale / errors")
    m = _lib()
    rng = np.random.default_rng(4)
    x = F.bf16_bits_from_f32((rng.standard_normal((1, 32, 64)) * 0.02).astype(np.float32))
    S = np.float32(0.0001234)
    q = m.quantize(dev_bf16(x), "nvfp4", "4over6", tensor_scale=torch.tensor([S]))
    o = Q.quantize_nvfp4(F.bf16_to_f64(x[0]), "4over6", tensor_scale=S)
    np.testing.assert_array_equal(host(q["codes"])[0], F.pack_nibbles(o["codes"]))
    np.testing.assert_array_equal(host(q["scales"])[0], o["scales"])
    with pytest.raises(m.Fp4Error):
        m.quantize(dev_bf16(x[:, :, :40]).contiguous(), "nvfp4")


@pytest.mark.parametrize("rule", ["4over6", "sweep"])
def test_nvfp4_large_batch_chunked_amax(rule):
    """A batch of 19 bf16 tensors of 1024 x 1024, large enough that the
    library takes each chunk's tensor amax inside the previous chunk's
    quantization launch.  Tensor scales must be the oracle's amax / 2688 of
    each tensor (amaxes differ by orders of magnitude across the batch and sit
    at scattered positions), codes and scales must match one-tensor calls
    bit for bit, and sampled rows must match the oracle."""
    print_case(f"nvfp4/{rule} 19 x 1024 x 1024 chunked amax")
    m = _lib()
    B, R, C = 19, 1024, 1024
    rng = np.random.default_rng(19)
    x = rng.standard_normal((B, R * C), dtype=np.float32)
    for b in range(B):
        x[b] *= np.float32(2.0 ** (b - 9) * (1 + 0.1 * b))
        x[b, (b * 104729 + 7) % (R * C)] = np.float32(7.5 * 2.0 ** (b - 9))
    bits = F.bf16_bits_from_f32(x).reshape(B, R, C)
    del x
    t = dev_bf16(bits)
    q = m.quantize(t, "nvfp4", rule)
    torch.cuda.synchronize()
    ts = host(q["tensor_scale"])
    codes, scales = host(q["codes"]), host(q["scales"])
    want_ts = [Q.nvfp4_tensor_scale(np.max(np.abs(F.bf16_to_f64(bits[b])))) for b in range(B)]
    for b in range(B):
        assert ts[b].view(np.uint32) == want_ts[b].view(np.uint32), f"tensor scale {b}"
    for b in (0, 9, 10, 18):
        one = m.quantize(t[b:b + 1], "nvfp4", rule)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes[b], host(one["codes"])[0], err_msg=f"codes, tensor {b}")
        np.testing.assert_array_equal(scales[b], host(one["scales"])[0], err_msg=f"scales, tensor {b}")
        rows = slice(64 * (b % 16), 64 * (b % 16) + 64)
        o = Q.quantize_nvfp4(F.bf16_to_f64(bits[b, rows]), rule, tensor_scale=want_ts[b])
        np.testing.assert_array_equal(codes[b, rows], F.pack_nibbles(o["codes"]), err_msg=f"oracle rows {b}")
        np.testing.assert_array_equal(scales[b, rows], o["scales"], err_msg=f"oracle scales {b}")


def test_nvfp4_eight_chunks_with_a_short_last_chunk():
    """67 bf16 tensors of 1024 x 1024: the batch is cut into 8 chunks of 9
    tensors (the last holds 4), each chunk's tensor amaxes taken inside the
    previous chunk's quantization launch (the streaming workload's path at
    512 experts).  Every tensor scale is the oracle's amax / 2688 bit for bit;
    codes and scales of the first and last tensor of every chunk equal
    one-tensor calls; two tensors' sampled rows equal the oracle."""
    print_case("nvfp4/4over6 67 x 1024 x 1024, 8 chunks")
    m = _lib()
    B, R, C = 67, 1024, 1024
    rng = np.random.default_rng(67)
    x = rng.standard_normal((B, R * C), dtype=np.float32)
    for b in range(B):
        x[b] *= np.float32(2.0 ** ((b % 23) - 11) * (1 + 0.01 * b))
        x[b, (b * 7919 + 13) % (R * C)] = np.float32(9.0 * 2.0 ** ((b % 23) - 11))
    bits = F.bf16_bits_from_f32(x).reshape(B, R, C)
    del x
    t = dev_bf16(bits)
    q = m.quantize(t, "nvfp4", "4over6")
    torch.cuda.synchronize()
    ts = host(q["tensor_scale"])
    want_ts = np.array([Q.nvfp4_tensor_scale(np.max(np.abs(F.bf16_to_f64(bits[b])))) for b in range(B)], np.float32)
    np.testing.assert_array_equal(ts.view(np.uint32), want_ts.view(np.uint32))
    codes, scales = host(q["codes"]), host(q["scales"])
    edges = sorted({b for c0 in range(0, B, 9) for b in (c0, min(c0 + 8, B - 1))})
    assert 63 in edges and 66 in edges
    for b in edges:
        one = m.quantize(t[b:b + 1], "nvfp4", "4over6")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes[b], host(one["codes"])[0], err_msg=f"codes, tensor {b}")
        np.testing.assert_array_equal(scales[b], host(one["scales"])[0], err_msg=f"scales, tensor {b}")
    for b in (8, 64):
        rows = slice(128, 192)
        o = Q.quantize_nvfp4(F.bf16_to_f64(bits[b, rows]), "4over6", tensor_scale=want_ts[b])
        np.testing.assert_array_equal(codes[b, rows], F.pack_nibbles(o["codes"]), err_msg=f"oracle rows {b}")
        np.testing.assert_array_equal(scales[b, rows], o["scales"], err_msg=f"oracle scales {b}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_error_matches_oracle(fmt, dtype):
    """fp4_block_error on three tensors (several 256-wide tiles of blocks)
    against the oracle's float64 block errors of its own 4/6 quantization of
    the same values; the GPU sums in f32 (each difference, square and sum
    rounded once), within 1e-5 relative per block."""
    m = _lib()
    print_case(f"block error {fmt} {dtype}")
    rng = np.random.default_rng(21)
    x32 = (rng.standard_t(4, size=(3, 40, 256)) * 0.02).astype(np.float32)
    if dtype == "bf16":
        bits = F.bf16_bits_from_f32(x32)
        xt, x64 = dev_bf16(bits), F.bf16_to_f64(bits)
    else:
        xt, x64 = dev(x32), x32.astype(np.float64)
    q = m.quantize(xt, fmt, "4over6")
    err = host(m.block_error(xt, q, fmt))
    bs = 16 if fmt == "nvfp4" else 32
    assert err.shape == (3, 40, 256 // bs)
    for b in range(3):
        qo = _oracle_q(fmt, x64[b], "4over6")
        xh = (Q.dequantize_nvfp4(qo["codes"], qo["scales"], qo["tensor_scale"]) if fmt == "nvfp4"
              else Q.dequantize_mxfp4(qo["codes"], qo["scales"]))
        ref = Q.block_sq_error(x64[b], xh, bs).reshape(40, 256 // bs)
        assert np.all(np.abs(err[b] - ref) <= 1e-5 * ref + 1e-30), f"tensor {b}"
