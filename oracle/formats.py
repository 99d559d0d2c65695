"""Exact codecs of the element and scale formats (oracle; test infrastructure only).

The cards name the formats but do not restate them: NVFP4 = E2M1 values with
one E4M3 scale per 16 values plus an FP32 tensor scale ("dabsLabs NVFP4",
section "What makes this build different"; "FP4-Local AZ", section "For
TensorFold": "NVFP4 group-16"), MXFP4 = E2M1 with UE8M0 microscales
("MXFP4-FP8-R12", section "Quantization format"), MXFP8 = E4M3 values with a
power-of-two scale per 32 ("FP4-Local AZ", section "The shared expert").
The bit layouts below are those formats' public definitions:

  E2M1  sign | 2 exponent bits (bias 1) | 1 mantissa bit.  Magnitudes of
        codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  E4M3  (FN variant) sign | 4 exponent bits (bias 7) | 3 mantissa bits;
        exponent field 0 is subnormal (m/8 * 2^-6); 0x7F / 0xFF are NaN; no
        infinities; largest finite value 448 (0x7E).
  UE8M0 unsigned exponent only: 2^(c - 127), c = 0..254; 0xFF is NaN.

Rounding is round-to-nearest with ties to the even code (the IEEE default),
saturating to the largest finite magnitude.  All values here are float64 and
every operation on them is exact for the operands that reach it.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0

# magnitudes of E2M1 codes 0..7 (code = e1 e0 m)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_decode(code) -> np.ndarray:
    """E4M3FN byte(s) -> float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


# the 127 finite non-negative E4M3 values, increasing with the code byte 0x00..0x7E
E4M3_GRID = e4m3_decode(np.arange(127))


def ue8m0_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def e2m1_decode(code) -> np.ndarray:
    """E2M1 nibble(s) (bit 3 = sign) -> float64."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def round_to_grid(a, unit, grid) -> np.ndarray:
    """Index of the grid value nearest to a/unit; ties to the even index; saturating.

    `a` (>= 0) and `unit` (> 0) are exact float64 values and `grid` is an
    increasing array of exactly representable values.  The decision is made
    by comparing `a` with each midpoint times `unit`; callers guarantee that
    every such product is exact in float64 (it has at most 53 significant
    bits), so no rounding enters the decision.  The index is the number of
    midpoints that `a` lies beyond, where lying exactly on a midpoint counts as
    beyond it iff the upper neighbour has an even index.
    """
    a = np.asarray(a, dtype=np.float64)
    unit = np.asarray(unit, dtype=np.float64)
    mids = (grid[1:] + grid[:-1]) / 2.0
    idx = np.zeros(np.broadcast(a, unit).shape, dtype=np.int64)
    for j, mid in enumerate(mids):
        t = mid * unit
        upper_even = (j + 1) % 2 == 0
        idx += (a > t) | ((a == t) & upper_even)
    return idx


def e4m3_encode(v) -> np.ndarray:
    """Non-negative float64 value(s) -> E4M3 code, RNE, saturating at 448 (satfinite)."""
    return round_to_grid(v, 1.0, E4M3_GRID).astype(np.uint8)


def e2m1_encode(x) -> np.ndarray:
    """float64 value(s) -> E2M1 nibble, RNE, saturating at 6; sign bit = sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    mag = round_to_grid(np.abs(x), 1.0, E2M1_GRID)
    return (mag | (np.signbit(x).astype(np.int64) << 3)).astype(np.uint8)


def bf16_bits_from_f32(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64: a bf16 value is the float32 whose
    upper 16 bits are its pattern and whose lower 16 bits are zero."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pack_nibbles(codes) -> np.ndarray:
    """[..., n] nibbles -> [..., n/2] bytes; element 2i in the low nibble, 2i+1 in the high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
