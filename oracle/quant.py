"""Quantizers and dequantizers (oracle; test infrastructure only).

Sources on block_scaled_fp4_nvfp4:
  * "dabsLabs NVFP4 (4/6-optimal scales)", section "What makes this build
    different": per 16-element block the scale is chosen between the amax/6
    plan and the four-over-six plan (block max mapped to 4) by exact
    post-rounding squared error; never worse than plain RTN.
  * "Local-Hessian NVFP4 experts", opening section: the activation
    input_scale is amax/2688 (not amax/6) and gate and up share one
    weight_scale_2; section "What is different about it": one
    weight_scale_2 per expert.
  * "FP4-Local AZ", section "The shared expert": MXFP8 = E4M3 values with one
    power-of-two scale per 32 weights, e = ceil(log2(amax / 448)).
  * "MXFP4-FP8-R12", section "Quantization format": MXFP4 E2M1 weights with
    UE8M0 microscales; activations dynamically quantized to MXFP8; retained
    layers in source block FP8.

Readings where the cards are silent (each is listed in the design notes):
  * blocks are contiguous along the last (input / reduction) dimension;
  * tensor scale S = fp32(fp64(amax) / 2688); S == 0 (all-zero tensor, or an
    f32 tensor whose amax/2688 underflows) gives scale bytes 0 and codes 0;
  * NVFP4 block scale of plan M: s_M = E4M3_RNE_satfinite(amax_b / (M * S));
  * E2M1 rounding is nearest, ties to the even code, saturating at 6; the
    sign nibble bit is the sign bit of x (so -0 encodes as 0x8);
  * the block error of a plan is sum_i (|x_i| - g_i * s_M * S)^2 in exact
    arithmetic; plan M=4 is chosen iff its error is strictly smaller;
  * the scale sweep (the "MSE sweep" the Local-Hessian card names in "What
    is different about it", without defining it) tries every E4M3 scale from
    the M=6 plan's to the M=4 plan's inclusive and keeps the first with the
    smallest exact post-rounding squared error; it contains both 4/6 plans,
    so its error never exceeds 4/6's;
  * the Hessian-weighted search (the "local_hessian" / H-Scale search the
    Local-Hessian card names in "What is different about it" and "Results",
    without defining it): the sweep's candidates, each block's error weighted
    by the 16 x 16 diagonal block H_b of the expert's input Hessian,
    err = d^T H_b d with d = x - xhat (signed), the first candidate with the
    smallest exact error kept; tensor scale amax/2688 unchanged; experts with
    fewer than 64 calibration rows take plain max (the amax/6 plan);
  * MXFP4 plan M: e_M = min{e : M * 2^e >= amax_b}, clamped to [-127, 127]
    (the no-clip ceiling rule, as in the MXFP8 rule of the AZ card);
  * block FP8: one fp32 scale sigma = fp32(amax / 448) per 128 x 128 weight
    tile or per (row, 128 columns) of activations; values E4M3_RNE_sat(x / sigma).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .formats import (E2M1_GRID, E4M3_GRID, E4M3_MAX, e2m1_decode,
                      e4m3_decode, e4m3_encode, round_to_grid)

NV_BLOCK = 16
MX_BLOCK = 32
FP8_TILE = 128
NV_TENSOR_DIVISOR = 2688.0  # 6 (E2M1 max) * 448 (E4M3 max)


def nvfp4_tensor_scale(amax) -> np.float32:
    """S = fp32(amax / 2688) ("Local-Hessian NVFP4 experts", opening section)."""
    return np.float32(np.float64(amax) / NV_TENSOR_DIVISOR)


def _blocks(x, size):
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % size:
        raise ValueError(f"last dimension {x.shape[-1]} is not a multiple of {size}")
    return x.reshape(-1, size)


def _exact_block_error(absx_row, g_row, unit) -> Fraction:
    u = Fraction(float(unit))
    return sum((Fraction(float(a)) - Fraction(float(g)) * u) ** 2
               for a, g in zip(absx_row, g_row))


def _plan(absx, unit):
    """E2M1 magnitude indices and float64 block errors for one scale plan.

    absx: [nblk, bs]; unit: [nblk] = scale value of the plan (0 allowed)."""
    safe = np.where(unit > 0, unit, 1.0)[:, None]
    mag = np.where(unit[:, None] > 0, round_to_grid(absx, safe, E2M1_GRID), 0)
    g = E2M1_GRID[mag]
    err = np.sum((absx - g * unit[:, None]) ** 2, axis=1)
    return mag, g, err


def _better(absx, unit_a, unit_b, plan_a, plan_b):
    """Boolean per block: True iff plan b has a strictly smaller exact error
    than plan a.

    The float64 errors decide unless they are within a relative 2^-40 of each
    other (their own rounding error is below 2^-48 relative); such near-ties
    are re-evaluated in exact rational arithmetic."""
    (_, ga, ea), (_, gb, eb) = plan_a, plan_b
    take = eb < ea
    # identical plans (same scale) tie exactly and keep plan a
    close = (np.abs(ea - eb) <= 2.0 ** -40 * (ea + eb)) & (unit_a != unit_b)
    for b in np.nonzero(close)[0]:
        xa = _exact_block_error(absx[b], ga[b], unit_a[b])
        xb = _exact_block_error(absx[b], gb[b], unit_b[b])
        take[b] = xb < xa
    return take


def _choose(absx, unit6, unit4, plan6, plan4):
    """Boolean per block: True iff plan M=4 has strictly smaller exact error."""
    return _better(absx, unit6, unit4, plan6, plan4)


def _sweep(absx, S, s6, s4, unit6, p6):
    """Scale sweep: every E4M3 code from the M=6 plan's to the M=4 plan's
    (E4M3 codes of non-negative values order like the values), the first
    with the smallest exact error wins.  Returns (codes, magnitude indices,
    offset of the chosen code from the M=6 plan's)."""
    width = s4.astype(np.int64) - s6.astype(np.int64)
    best_s = s6.astype(np.int64)
    best_unit = unit6
    best = p6
    choice = np.zeros(len(s6), np.int64)
    for off in range(1, int(width.max(initial=0)) + 1):
        live = off <= width
        cand = np.where(live, s6.astype(np.int64) + off, s6.astype(np.int64))
        unit = e4m3_decode(cand) * S
        pc = _plan(absx, unit)
        take = _better(absx, best_unit, unit, best, pc) & live
        best_s = np.where(take, cand, best_s)
        best_unit = np.where(take, unit, best_unit)
        best = (np.where(take[:, None], pc[0], best[0]), np.where(take[:, None], pc[1], best[1]),
                np.where(take, pc[2], best[2]))
        choice = np.where(take, off, choice)
    return best_s.astype(np.uint8), best[0], choice


def quantize_nvfp4(x, rule: str = "4over6", tensor_scale=None):
    """NVFP4 quantization of one tensor [..., cols] (cols % 16 == 0).

    Returns dict: codes (uint8 nibbles, same shape as x), scales (uint8 E4M3,
    [..., cols/16]), tensor_scale (float32), m4 (bool per block: plan M=4
    chosen; for the sweep, a scale other than the M=6 plan's), and for the
    sweep `choice` (offset of the chosen E4M3 code from the M=6 plan's).
    """
    x = np.asarray(x, dtype=np.float64)
    blk = _blocks(x, NV_BLOCK)
    absx = np.abs(blk)
    if tensor_scale is None:
        tensor_scale = nvfp4_tensor_scale(np.max(absx) if absx.size else 0.0)
    S = np.float64(np.float32(tensor_scale))
    amax_b = np.max(absx, axis=1)

    def plan_scale(M):
        if S == 0.0:
            return np.zeros(len(amax_b), np.uint8)
        return e4m3_encode(amax_b / (M * S))

    s6 = plan_scale(6.0)
    unit6 = e4m3_decode(s6) * S
    p6 = _plan(absx, unit6)
    if rule == "rtn":
        choose4 = np.zeros(len(amax_b), bool)
        s4, p4 = s6, p6
    elif rule == "4over6":
        s4 = plan_scale(4.0)
        unit4 = e4m3_decode(s4) * S
        p4 = _plan(absx, unit4)
        choose4 = _choose(absx, unit6, unit4, p6, p4)
    elif rule == "sweep":
        scales, mag, choice = _sweep(absx, S, s6, plan_scale(4.0), unit6, p6)
        codes = (mag | (np.signbit(blk).astype(np.int64) << 3)).astype(np.uint8)
        shp = x.shape[:-1] + (x.shape[-1] // NV_BLOCK,)
        return {"codes": codes.reshape(x.shape), "scales": scales.reshape(shp), "tensor_scale": np.float32(S),
                "m4": (choice > 0).reshape(shp), "choice": choice.astype(np.uint8).reshape(shp)}
    else:
        raise ValueError(rule)
    mag = np.where(choose4[:, None], p4[0], p6[0])
    codes = (mag | (np.signbit(blk).astype(np.int64) << 3)).astype(np.uint8)
    scales = np.where(choose4, s4, s6).astype(np.uint8)
    return {
        "codes": codes.reshape(x.shape),
        "scales": scales.reshape(x.shape[:-1] + (x.shape[-1] // NV_BLOCK,)),
        "tensor_scale": np.float32(S),
        "m4": choose4.reshape(x.shape[:-1] + (x.shape[-1] // NV_BLOCK,)),
    }


HESSIAN_MIN_ROWS = 64  # "experts with a full Hessian (>= 64 routed rows)"


def _exact_weighted_error(x_row, q_row, H) -> Fraction:
    """sum_ij H_ij d_i d_j with d = x - q, in exact rational arithmetic."""
    d = [Fraction(float(a)) - Fraction(float(b)) for a, b in zip(x_row, q_row)]
    Hf = [[Fraction(float(v)) for v in row] for row in H]
    return sum(Hf[i][j] * d[i] * d[j] for i in range(len(d)) for j in range(len(d)))


def quantize_nvfp4_hessian(x, hessian, calib_rows: int, tensor_scale=None):
    """NVFP4 quantization of one expert matrix x [rows, cols] (cols % 16 == 0)
    with block scales chosen by a Hessian-weighted search.

    Local-Hessian NVFP4 card, "What is different about it": the per-group
    weight scales come from a Hessian-weighted search ("local_hessian",
    H-Scale) instead of the plain amax/MSE sweep, and only the weight_scale
    values differ (same format, same tensor scale); "Results": experts with a
    full Hessian have >= 64 routed calibration rows, thinner ones (including
    none) keep plain max.  The search itself is not defined on the pages.
    Reading:
      * hessian [cols/16, 16, 16]: H_b, the diagonal 16 x 16 block of the
        expert's input Hessian (1/n) sum_t a_t a_t^T for the columns of block b
        (the output error of a block of row r over the calibration rows is
        d^T H_b d, cross-block terms left out: "local");
      * candidates: every E4M3 scale code from the amax/6 plan's to the
        block-max-to-4 plan's, in increasing order (the sweep's window),
        codes by E2M1 round-to-nearest-even of x / (s * S);
      * err = sum_ij H_b[i, j] d_i d_j with d = x - xhat signed; the first
        candidate with the smallest exact err is kept;
      * calib_rows < 64: the amax/6 plan (plain max) for every block.
    The float64 errors decide unless two are within 2^-40 of the sum of
    sum_ij |H_ij| |d_i| |d_j| of both (their rounding error is below 2^-47 of
    it); those are decided in exact rational arithmetic.
    Returns dict: codes (nibbles [rows, cols]), scales (uint8 [rows, cols/16]),
    tensor_scale (float32), choice (uint8 [rows, cols/16]: chosen code minus
    the amax/6 plan's)."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    if C % NV_BLOCK:
        raise ValueError("cols must be a multiple of 16")
    if calib_rows < HESSIAN_MIN_ROWS:
        q = quantize_nvfp4(x, "rtn", tensor_scale)
        q["choice"] = np.zeros(q["scales"].shape, np.uint8)
        return q
    H = np.asarray(hessian, dtype=np.float64)
    nb = C // NV_BLOCK
    if H.shape != (nb, NV_BLOCK, NV_BLOCK):
        raise ValueError("hessian must be [cols/16, 16, 16]")
    blk = x.reshape(-1, NV_BLOCK)
    absx = np.abs(blk)
    sgn = np.where(np.signbit(blk), -1.0, 1.0)
    Hb = np.broadcast_to(H[None], (R, nb, NV_BLOCK, NV_BLOCK)).reshape(-1, NV_BLOCK, NV_BLOCK)
    absH = np.abs(Hb)
    if tensor_scale is None:
        tensor_scale = nvfp4_tensor_scale(np.max(absx) if absx.size else 0.0)
    S = np.float64(np.float32(tensor_scale))
    amax_b = np.max(absx, axis=1)

    def plan_scale(M):
        if S == 0.0:
            return np.zeros(len(amax_b), np.int64)
        return e4m3_encode(amax_b / (M * S)).astype(np.int64)

    def candidate(code):
        unit = e4m3_decode(code) * S
        safe = np.where(unit > 0, unit, 1.0)[:, None]
        mag = np.where(unit[:, None] > 0, round_to_grid(absx, safe, E2M1_GRID), 0)
        q = sgn * E2M1_GRID[mag] * unit[:, None]          # exact (<= 31 significant bits)
        d = blk - q                                       # exact (see the design notes)
        err = np.einsum("ni,nij,nj->n", d, Hb, d)
        bound = np.einsum("ni,nij,nj->n", np.abs(d), absH, np.abs(d))
        return mag, q, err, bound

    s6, s4 = plan_scale(6.0), plan_scale(4.0)
    best_code = s6.copy()
    best_mag, best_q, best_err, best_bound = candidate(s6)
    width = s4 - s6
    for off in range(1, int(width.max(initial=0)) + 1):
        live = off <= width
        code = np.where(live, s6 + off, s6)
        mag, q, err, bound = candidate(code)
        take = err < best_err
        close = np.abs(err - best_err) <= 2.0 ** -40 * (bound + best_bound)
        for b in np.nonzero(close & live)[0]:
            hb = H[b % nb]
            take[b] = _exact_weighted_error(blk[b], q[b], hb) < _exact_weighted_error(blk[b], best_q[b], hb)
        take &= live
        best_code = np.where(take, code, best_code)
        best_mag = np.where(take[:, None], mag, best_mag)
        best_q = np.where(take[:, None], q, best_q)
        best_err = np.where(take, err, best_err)
        best_bound = np.where(take, bound, best_bound)
    codes = (best_mag | (np.signbit(blk).astype(np.int64) << 3)).astype(np.uint8)
    return {"codes": codes.reshape(R, C), "scales": best_code.astype(np.uint8).reshape(R, nb),
            "tensor_scale": np.float32(S), "choice": (best_code - s6).astype(np.uint8).reshape(R, nb)}


def hessian_weighted_error(x, codes, scales, tensor_scale, hessian) -> np.ndarray:
    """Per-block d^T H_b d (float64) of a quantization of x [rows, cols]: the
    quantity the Hessian-weighted search minimizes, for reporting."""
    x = np.asarray(x, np.float64)
    R, C = x.shape
    d = (x - dequantize_nvfp4(codes, scales, tensor_scale)).reshape(R, C // NV_BLOCK, NV_BLOCK)
    return np.einsum("rbi,bij,rbj->rb", d, np.asarray(hessian, np.float64), d)


def dequantize_nvfp4(codes, scales, tensor_scale) -> np.ndarray:
    """Exact values g * s * S in float64 (g E2M1, s E4M3, S fp32); the product
    has at most 31 significant bits, so float64 holds it exactly."""
    g = e2m1_decode(codes)
    s = np.repeat(e4m3_decode(scales), NV_BLOCK, axis=-1)
    return g * s * np.float64(np.float32(tensor_scale))


def min_pow2_exponent(a, M) -> np.ndarray:
    """Smallest integer e with M * 2^e >= a (a > 0), by exact comparisons."""
    a = np.asarray(a, dtype=np.float64)
    _, p = np.frexp(a)           # a in [2^(p-1), 2^p)
    e = p.astype(np.int64) - 12  # below the answer for every M <= 2^10
    for _ in range(16):
        e = np.where(np.ldexp(np.float64(M), e) < a, e + 1, e)
    return e


def _mx_exponent(amax_b, M):
    e = np.where(amax_b > 0, min_pow2_exponent(np.where(amax_b > 0, amax_b, 1.0), M), -127)
    return np.clip(e, -127, 127)


def quantize_mxfp4(x, rule: str = "4over6"):
    """MXFP4 quantization of [..., cols] (cols % 32 == 0).

    Returns dict: codes (nibbles), scales (uint8 UE8M0, [..., cols/32]), m4."""
    x = np.asarray(x, dtype=np.float64)
    blk = _blocks(x, MX_BLOCK)
    absx = np.abs(blk)
    amax_b = np.max(absx, axis=1)
    e6 = _mx_exponent(amax_b, 6.0)
    unit6 = np.ldexp(1.0, e6)
    p6 = _plan(absx, unit6)
    if rule == "rtn":
        choose4 = np.zeros(len(amax_b), bool)
        e4, p4 = e6, p6
    elif rule == "4over6":
        e4 = _mx_exponent(amax_b, 4.0)
        unit4 = np.ldexp(1.0, e4)
        p4 = _plan(absx, unit4)
        choose4 = _choose(absx, unit6, unit4, p6, p4)
    elif rule == "sweep":
        # every power-of-two scale from the M=6 plan's to the M=4 plan's, the
        # first with the smallest exact error (4/6 < 2, so at most two exist)
        e4 = _mx_exponent(amax_b, 4.0)
        best_e, best_unit, best = e6.copy(), unit6, p6
        for off in range(1, int(np.max(e4 - e6, initial=0)) + 1):
            live = off <= e4 - e6
            cand = np.where(live, e6 + off, e6)
            unit = np.ldexp(1.0, cand)
            pc = _plan(absx, unit)
            take = _better(absx, best_unit, unit, best, pc) & live
            best_e = np.where(take, cand, best_e)
            best_unit = np.where(take, unit, best_unit)
            best = (np.where(take[:, None], pc[0], best[0]), np.where(take[:, None], pc[1], best[1]),
                    np.where(take, pc[2], best[2]))
        choose4 = best_e != e6
        e4, p4 = best_e, best
    else:
        raise ValueError(rule)
    mag = np.where(choose4[:, None], p4[0], p6[0])
    codes = (mag | (np.signbit(blk).astype(np.int64) << 3)).astype(np.uint8)
    scales = (np.where(choose4, e4, e6) + 127).astype(np.uint8)
    return {
        "codes": codes.reshape(x.shape),
        "scales": scales.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK,)),
        "m4": choose4.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK,)),
    }


def dequantize_mxfp4(codes, scales) -> np.ndarray:
    g = e2m1_decode(codes)
    e = np.repeat(np.asarray(scales, dtype=np.int64) - 127, MX_BLOCK, axis=-1)
    return np.ldexp(g, e)


def quantize_mxfp8(x):
    """MXFP8 of [..., cols]: per 32 values e = min{e : 448 * 2^e >= amax}
    (= ceil(log2(amax/448)), "FP4-Local AZ", section "The shared expert"),
    values E4M3_RNE_satfinite(x * 2^-e).  Zero block: scale byte 0 (e = -127).

    Returns dict: codes (uint8 E4M3), scales (uint8 UE8M0, [..., cols/32])."""
    x = np.asarray(x, dtype=np.float64)
    blk = _blocks(x, MX_BLOCK)
    absx = np.abs(blk)
    e = _mx_exponent(np.max(absx, axis=1), E4M3_MAX)
    scaled = np.ldexp(absx, -e[:, None])  # exact: multiplication by a power of two
    mag = round_to_grid(scaled, 1.0, E4M3_GRID)
    codes = (mag | (np.signbit(blk).astype(np.int64) << 7)).astype(np.uint8)
    return {
        "codes": codes.reshape(x.shape),
        "scales": (e + 127).astype(np.uint8).reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK,)),
    }


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    v = e4m3_decode(codes)
    e = np.repeat(np.asarray(scales, dtype=np.int64) - 127, MX_BLOCK, axis=-1)
    return np.ldexp(v, e)


def fp8_scale(amax) -> np.ndarray:
    """sigma = fp32(fp64(amax) / 448)."""
    return (np.asarray(amax, dtype=np.float64) / E4M3_MAX).astype(np.float32)


def _e4m3_scaled(absx, sigma):
    """E4M3 indices of |x| / sigma (sigma fp32 > 0): compares with midpoint*sigma,
    exact in float64 (5 + 24 significant bits)."""
    return round_to_grid(absx, sigma, E4M3_GRID)


def quantize_fp8_block_weight(w, tile: int = FP8_TILE):
    """Block FP8 of a weight [rows, cols]: one fp32 scale per tile x tile block.

    Returns dict: codes (uint8 E4M3 [rows, cols]), scales (float32 [rows/tile, cols/tile])."""
    w = np.asarray(w, dtype=np.float64)
    R, C = w.shape
    if R % tile or C % tile:
        raise ValueError("weight dims must be multiples of the tile")
    t = w.reshape(R // tile, tile, C // tile, tile)
    amax = np.max(np.abs(t), axis=(1, 3))
    sigma = fp8_scale(amax)
    sig = np.float64(1.0) * sigma[:, None, :, None]
    safe = np.where(sig > 0, sig, 1.0)
    mag = np.where(sig > 0, _e4m3_scaled(np.abs(t), safe), 0)
    codes = (mag | (np.signbit(t).astype(np.int64) << 7)).astype(np.uint8)
    return {"codes": codes.reshape(R, C), "scales": sigma}


def dequantize_fp8_block_weight(codes, scales, tile: int = FP8_TILE) -> np.ndarray:
    v = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), tile, axis=0), tile, axis=1)
    return v * s


def quantize_fp8_rows(x, group: int = FP8_TILE):
    """Block FP8 of activations [rows, cols]: one fp32 scale per (row, group columns).

    Returns dict: codes (uint8 E4M3), scales (float32 [rows, cols/group])."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    if C % group:
        raise ValueError("cols must be a multiple of the group")
    t = x.reshape(R, C // group, group)
    sigma = fp8_scale(np.max(np.abs(t), axis=2))
    sig = np.float64(1.0) * sigma[:, :, None]
    safe = np.where(sig > 0, sig, 1.0)
    mag = np.where(sig > 0, _e4m3_scaled(np.abs(t), safe), 0)
    codes = (mag | (np.signbit(t).astype(np.int64) << 7)).astype(np.uint8)
    return {"codes": codes.reshape(R, C), "scales": sigma}


def dequantize_fp8_rows(codes, scales, group: int = FP8_TILE) -> np.ndarray:
    v = e4m3_decode(codes)
    return v * np.repeat(np.asarray(scales, np.float64), group, axis=1)


def block_sq_error(x, xhat, size) -> np.ndarray:
    """Per-block squared reconstruction error sum_i (x_i - xhat_i)^2 in
    float64, blocks of `size` consecutive values along the last dimension:
    the quantity the 4/6 rule compares ("dabsLabs NVFP4", section "What makes
    this build different"), reported per block."""
    d = (np.asarray(x, np.float64) - np.asarray(xhat, np.float64)).reshape(-1, size)
    return np.sum(d * d, axis=1)
