"""Pins of the oracle's format codecs against independent references.

E4M3 and UE8M0 are checked against torch's float8_e4m3fn / float8_e8m0fnu
dtypes (an independent implementation of the same formats); E2M1 and scaled
rounding are checked by brute force in exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    # landmarks of the format definition
    assert F.e4m3_decode(0x7E) == 448.0 and F.e4m3_decode(0x01) == 2.0 ** -9
    assert F.e4m3_decode(0x38) == 1.0 and F.e4m3_decode(0x08) == 2.0 ** -6
    assert np.all(np.diff(F.E4M3_GRID) > 0) and len(F.E4M3_GRID) == 127


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    grid = F.E4M3_GRID
    mids = (grid[1:] + grid[:-1]) / 2
    v = np.concatenate([
        grid, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
        np.exp2(rng.uniform(-12, np.log2(464), 20000)).astype(np.float32).astype(np.float64),
        [0.0, 448.0, 450.0, 464.0]])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch rounds float32; compare only where float32 holds v exactly
    exact = v.astype(np.float32).astype(np.float64) == v
    np.testing.assert_array_equal(F.e4m3_encode(v)[exact], ref[exact])
    # saturating beyond the last midpoint (torch returns NaN there)
    assert np.all(F.e4m3_encode(np.array([465.0, 480.0, 1e30])) == 0x7E)


def test_ue8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = F.ue8m0_decode(codes)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[:255], ref[:255])


def _brute_nearest(a, unit, grid):
    """Index of the nearest grid*unit to a by enumeration in exact rationals; ties to even index."""
    a, unit = Fraction(float(a)), Fraction(float(unit))
    d = [abs(a - Fraction(float(g)) * unit) for g in grid]
    best = min(d)
    cands = [i for i, di in enumerate(d) if di == best]
    if len(cands) == 1:
        return cands[0]
    assert len(cands) == 2
    return cands[0] if cands[0] % 2 == 0 else cands[1]


def test_e2m1_encode_brute_force_and_ties():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, code in ties.items():
        assert F.e2m1_encode(v) == code and F.e2m1_encode(-v) == code | 8
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.uniform(0, 7, 3000), F.E2M1_GRID, [6.5, 100.0]])
    for v in vals:
        want = min(_brute_nearest(v, 1.0, F.E2M1_GRID), 7)
        assert F.e2m1_encode(v) == want, v
    assert F.e2m1_encode(-0.0) == 8 and F.e2m1_encode(0.0) == 0


def test_scaled_rounding_brute_force_exact():
    """round_to_grid(a, s*S) against exact enumeration for E4M3 s and fp32 S."""
    rng = np.random.default_rng(2)
    for _ in range(3000):
        S = np.float64(np.float32(rng.uniform(1e-6, 1.0)))
        s = F.E4M3_GRID[rng.integers(1, 127)]
        unit = s * S
        g = F.E2M1_GRID[rng.integers(0, 8)]
        # values at, next to and between the decision points
        a = np.float64(np.float32(g * unit * rng.choice([1.0, 1 + 1e-7, 1 - 1e-7, rng.uniform(0.5, 1.5)])))
        got = int(F.round_to_grid(a, unit, F.E2M1_GRID))
        assert got == _brute_nearest(a, unit, F.E2M1_GRID), (a, unit)
    # exact midpoint ties in scaled units
    for S in (np.float64(np.float32(1 / 3)), 1.0, np.float64(np.float32(0.0123))):
        for s in (1.375, 448.0, 2.0 ** -9):
            unit = s * S
            for j, mid in enumerate((F.E2M1_GRID[1:] + F.E2M1_GRID[:-1]) / 2):
                a = mid * unit
                assert int(F.round_to_grid(a, unit, F.E2M1_GRID)) == _brute_nearest(a, unit, F.E2M1_GRID)


def test_nibble_order_and_roundtrip():
    # element 2i -> low nibble, element 2i+1 -> high nibble
    assert F.pack_nibbles(np.array([1, 2], np.uint8))[0] == 0x21
    c = np.random.default_rng(3).integers(0, 16, (5, 64)).astype(np.uint8)
    np.testing.assert_array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)


def test_bf16_rne():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], np.float32)
    # ties go to even mantissa; above the tie rounds up
    np.testing.assert_array_equal(F.bf16_bits_from_f32(v), [0x3F80, 0x3F80, 0x3F82, 0x3F81])
    ref = torch.from_numpy(np.random.default_rng(4).standard_normal(10000).astype(np.float32))
    np.testing.assert_array_equal(F.bf16_bits_from_f32(ref.numpy()),
                                  ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def _bf16_decoder_pins_hold(dec):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        ours = dec(bits)
    finite = np.isfinite(ref)
    ok = np.array_equal(np.isnan(ours), np.isnan(ref))
    ok &= np.array_equal(ours[finite], ref[finite]) and np.array_equal(ours[np.isinf(ref)], ref[np.isinf(ref)])
    # landmarks of the format: 1, -2, the largest finite value, the smallest subnormal, -0
    ok &= dec(np.uint16(0x3F80)) == 1.0 and dec(np.uint16(0xC000)) == -2.0
    ok &= dec(np.uint16(0x7F7F)) == (2.0 - 2.0 ** -7) * 2.0 ** 127
    ok &= dec(np.uint16(0x0001)) == 2.0 ** -133
    ok &= bool(np.signbit(dec(np.uint16(0x8000))))
    return bool(ok)


def test_bf16_decode_all_patterns():
    """bf16_to_f64 against torch's bfloat16 -> float64 conversion on all 65,536
    bit patterns (NaN patterns only checked to decode as NaN)."""
    assert _bf16_decoder_pins_hold(F.bf16_to_f64)
    # planted mistakes each fail: a wrong shift, the pattern's bytes swapped
    assert not _bf16_decoder_pins_hold(
        lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64))
    assert not _bf16_decoder_pins_hold(
        lambda b: (np.asarray(b, np.uint16).byteswap().astype(np.uint32) << 16).view(np.float32)
        .astype(np.float64))
