"""Pins of the oracle's Hessian-weighted NVFP4 scale search
(oracle/quant.py::quantize_nvfp4_hessian; Local-Hessian NVFP4 card, "What is
different about it" and "Results").

The search is pinned by: hand-worked blocks (tests/golden/
hessian_worked_example.txt), its reduction to the plain scale sweep when
H = c * I, an independent enumeration over the candidate window in exact
rationals, the thin-expert rule (< 64 calibration rows: plain max), the
never-worse property against plain max and 4/6 under the weighted error,
invariances, and planted mistakes that each fail one of them."""
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hessian_worked_example.txt")


def _golden():
    out = {}
    with open(GOLDEN) as f:
        lines = f.readlines()
    for line in lines:
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def _fr(v):
    return Fraction(float(v))


def _nearest_e4m3(q: Fraction) -> int:
    """E4M3 code nearest to q >= 0 by enumeration; ties to the even code; saturating."""
    if q >= 448:
        return 0x7E
    d = [abs(q - _fr(g)) for g in F.E4M3_GRID]
    best = min(d)
    c = [i for i, x in enumerate(d) if x == best]
    return c[0] if len(c) == 1 or c[0] % 2 == 0 else c[1]


def _nearest_e2m1(a: Fraction, unit: Fraction) -> int:
    d = [abs(a - _fr(g) * unit) for g in F.E2M1_GRID]
    best = min(d)
    c = [i for i, x in enumerate(d) if x == best]
    return c[0] if len(c) == 1 or c[0] % 2 == 0 else c[1]


def _brute_block(x, H, S: Fraction, weighted=True, signed=True, first=True):
    """(scale code, E2M1 magnitude codes, offset) of one block by enumeration
    in exact rationals.  The keyword switches plant the mistakes the negative
    controls check for."""
    xs = [_fr(v) for v in x]
    amax = max(abs(v) for v in xs)
    if S == 0 or amax == 0:
        return 0, [0] * len(xs), 0
    c6, c4 = _nearest_e4m3(amax / (6 * S)), _nearest_e4m3(amax / (4 * S))
    Hf = [[_fr(v) for v in row] for row in H]
    best = None
    for c in range(c6, c4 + 1):
        u = _fr(F.E4M3_GRID[c]) * S
        mags = [_nearest_e2m1(abs(v), u) for v in xs]
        if signed:
            d = [v - (1 if v >= 0 and not np.signbit(float(v)) else -1) * _fr(F.E2M1_GRID[m]) * u
                 for v, m in zip(xs, mags)]
        else:
            d = [abs(v) - _fr(F.E2M1_GRID[m]) * u for v, m in zip(xs, mags)]
        n = len(d)
        if weighted:
            err = sum(Hf[i][j] * d[i] * d[j] for i in range(n) for j in range(n))
        else:
            err = sum(Hf[i][i] * d[i] * d[i] for i in range(n))
        if best is None or err < best[1] or (not first and err == best[1]):
            best = (c, err, mags, c - c6)
    return best[0], best[2], best[3]


def _golden_blocks():
    """The four hand-worked blocks as one row of 64 values with their H blocks."""
    g = _golden()
    x = np.zeros((1, 64))
    H = np.stack([np.eye(16) for _ in range(4)])
    for b, name in enumerate("ABCD"):
        vals = [float(v) for v in g[f"{name}_x"]]
        x[0, 16 * b:16 * b + len(vals)] = vals
    H[0, 0, 1] = H[0, 1, 0] = float(g["A_h01"][0])
    H[1, 0, 1] = H[1, 1, 0] = float(g["B_h01"][0])
    H[2] = 0.0
    H[2, 0, 0] = 1.0
    H[3] = 0.0
    H[3, :2, :2] = [[1.0, -1.0], [-1.0, 1.0]]
    H[3, 2, 2] = 2.0 ** -50
    return g, x, H.astype(np.float32)


def test_hessian_worked_example():
    g, x, H = _golden_blocks()
    q = Q.quantize_nvfp4_hessian(x, H, 100, tensor_scale=np.float32(1.0))
    sc, ch, codes = q["scales"][0], q["choice"][0], q["codes"][0]
    assert sc[0] == int(g["A_scale"][0], 16) and ch[0] == int(g["A_choice"][0])
    np.testing.assert_array_equal(codes[0:2], [int(v) for v in g["A_codes01"]])
    assert sc[1] == int(g["B_scale"][0], 16)
    np.testing.assert_array_equal(codes[16:18], [int(v) for v in g["B_codes01"]])
    assert sc[2] == int(g["C_scale"][0], 16) and ch[2] == int(g["C_choice"][0])
    np.testing.assert_array_equal(codes[32:34], [int(v) for v in g["C_codes01"]])
    assert sc[3] == int(g["D_scale"][0], 16)
    np.testing.assert_array_equal(codes[48:51], [int(v) for v in g["D_codes012"]])
    # the zeros of every block encode as +0
    assert np.all(codes[2:16] == 0) and np.all(codes[51:64] == 0)
    # the plain sweep (H = I) picks the 4/6 plan on block A, as the fixture states
    assert Q.quantize_nvfp4(x[:, :16], "sweep", tensor_scale=np.float32(1.0))["scales"][0, 0] == \
        int(g["A_scale_diagonal_only"][0], 16)


def test_hessian_worked_example_planted_mistakes_fail():
    """The fixture's alternative answers are what each plausible mistake gives:
    the diagonal of H only (block A), unsigned residuals (block B), keeping
    the last of equal errors (block C)."""
    g, x, H = _golden_blocks()
    S = Fraction(1)
    diag_only = _brute_block(x[0, 0:16], H[0], S, weighted=False)[0]
    assert diag_only == int(g["A_scale_diagonal_only"][0], 16) != int(g["A_scale"][0], 16)
    unsigned = _brute_block(x[0, 16:32], H[1], S, signed=False)[0]
    assert unsigned == int(g["B_scale_unsigned_residuals"][0], 16) != int(g["B_scale"][0], 16)
    last = _brute_block(x[0, 32:48], H[2], S, first=False)[0]
    assert last == int(g["C_scale_last_minimum"][0], 16) != int(g["C_scale"][0], 16)
    # and the correct enumeration reproduces the fixture on all four blocks
    for b, name in enumerate("ABCD"):
        assert _brute_block(x[0, 16 * b:16 * b + 16], H[b], S)[0] == int(g[f"{name}_scale"][0], 16)


def _bf16(rng, shape, std=0.02, heavy=False):
    v = rng.standard_t(4, shape) if heavy else rng.standard_normal(shape)
    return F.bf16_to_f64(F.bf16_bits_from_f32((v * std).astype(np.float32)))


@pytest.mark.parametrize("heavy", [False, True])
def test_hessian_identity_reduces_to_the_sweep(heavy):
    """H = c * I weights every value alike: the search is the plain sweep."""
    rng = np.random.default_rng(20 + heavy)
    x = _bf16(rng, (16, 128), heavy=heavy)
    ref = Q.quantize_nvfp4(x, "sweep")
    for c in (1.0, 3.0, 2.0 ** -20):
        H = np.stack([np.eye(16, dtype=np.float32) * np.float32(c)] * 8)
        q = Q.quantize_nvfp4_hessian(x, H, 64)
        np.testing.assert_array_equal(q["codes"], ref["codes"])
        np.testing.assert_array_equal(q["scales"], ref["scales"])
        np.testing.assert_array_equal(q["choice"], ref["choice"])
        assert q["tensor_scale"] == ref["tensor_scale"]


@pytest.mark.parametrize("seed,heavy", [(30, False), (31, True)])
def test_hessian_matches_exact_brute_force(seed, heavy):
    rng = np.random.default_rng(seed)
    x = _bf16(rng, (6, 64), heavy=heavy)
    H = synth.calibration_hessian(seed, 0, 64, 96)
    q = Q.quantize_nvfp4_hessian(x, H, 96)
    S = _fr(np.float32(np.float64(np.max(np.abs(x))) / 2688.0))
    assert _fr(q["tensor_scale"]) == S
    differs_from_sweep = 0
    sweep = Q.quantize_nvfp4(x, "sweep")
    for r in range(x.shape[0]):
        for b in range(4):
            blk = x[r, 16 * b:16 * b + 16]
            c, mags, off = _brute_block(blk, H[b], S)
            assert q["scales"][r, b] == c and q["choice"][r, b] == off, (r, b)
            want = np.array(mags) | (np.signbit(blk).astype(int) << 3)
            np.testing.assert_array_equal(q["codes"][r, 16 * b:16 * b + 16], want)
            differs_from_sweep += c != sweep["scales"][r, b]
    assert differs_from_sweep > 0   # the weighting changes some choices on this data


def test_hessian_exact_near_ties():
    """Blocks whose candidates' errors differ far below the float64 rounding of
    the cancelling terms (block D of the fixture, scaled into every row) are
    decided exactly."""
    g, x0, H = _golden_blocks()
    rng = np.random.default_rng(40)
    rows = []
    for _ in range(12):
        r = np.zeros(16)
        a = float(rng.choice([4.5, 5.5, 6.0, 7.0]))
        r[0] = r[1] = a
        r[2] = float(F.bf16_to_f64(F.bf16_bits_from_f32(np.array([rng.uniform(0.05, 0.9)], np.float32)))[0])
        rows.append(r)
    x = np.stack(rows)
    Hd = H[3:4]
    q = Q.quantize_nvfp4_hessian(x, Hd, 64, tensor_scale=np.float32(1.0))
    for i in range(x.shape[0]):
        c, mags, off = _brute_block(x[i], Hd[0], Fraction(1))
        assert q["scales"][i, 0] == c and q["choice"][i, 0] == off
        np.testing.assert_array_equal(q["codes"][i], mags)


def test_hessian_thin_experts_take_plain_max():
    rng = np.random.default_rng(50)
    x = _bf16(rng, (8, 64), heavy=True)
    H = synth.calibration_hessian(50, 0, 64, 200)
    rtn = Q.quantize_nvfp4(x, "rtn")
    for n in (0, 1, 63):
        q = Q.quantize_nvfp4_hessian(x, H, n)
        np.testing.assert_array_equal(q["codes"], rtn["codes"])
        np.testing.assert_array_equal(q["scales"], rtn["scales"])
        assert not q["choice"].any()
    q64 = Q.quantize_nvfp4_hessian(x, H, 64)
    assert (q64["scales"] != rtn["scales"]).any()


def test_hessian_never_worse_than_plain_max_or_four_over_six():
    """Both the amax/6 plan and the 4/6 choice are in the window, so the
    chosen scale's weighted error is at most theirs (exact rationals)."""
    rng = np.random.default_rng(60)
    x = _bf16(rng, (4, 128), heavy=True)
    H = synth.calibration_hessian(60, 0, 128, 80)
    q = Q.quantize_nvfp4_hessian(x, H, 80)
    S = q["tensor_scale"]
    others = [Q.quantize_nvfp4(x, rule) for rule in ("rtn", "4over6")]

    def werr(qq, r, b):
        xh = Q.dequantize_nvfp4(qq["codes"][r, 16 * b:16 * b + 16], qq["scales"][r, b:b + 1], S)
        d = [_fr(a) - _fr(c) for a, c in zip(x[r, 16 * b:16 * b + 16], xh)]
        return sum(_fr(H[b][i][j]) * d[i] * d[j] for i in range(16) for j in range(16))

    strict = 0
    for r in range(4):
        for b in range(8):
            e = werr(q, r, b)
            eo = [werr(o, r, b) for o in others]
            assert all(e <= v for v in eo)
            strict += e < min(eo)
    assert strict > 0


def test_hessian_invariances():
    rng = np.random.default_rng(70)
    x = _bf16(rng, (8, 64))
    H = synth.calibration_hessian(70, 0, 64, 120)
    q = Q.quantize_nvfp4_hessian(x, H, 120)
    # a positive multiple of H ranks the candidates alike
    for c in (0.37, 5.0):
        qc = Q.quantize_nvfp4_hessian(x, (H * np.float32(c)).astype(np.float32), 120)
        np.testing.assert_array_equal(qc["codes"], q["codes"])
        np.testing.assert_array_equal(qc["scales"], q["scales"])
    # powers of two on x: same codes and scales (S scales with x)
    for j in (-6, 3):
        qj = Q.quantize_nvfp4_hessian(np.ldexp(x, j), H, 120)
        np.testing.assert_array_equal(qj["codes"], q["codes"])
        np.testing.assert_array_equal(qj["scales"], q["scales"])
    # sign flip: d^T H d is even in d, so only the sign bits change
    qn = Q.quantize_nvfp4_hessian(-x, H, 120)
    np.testing.assert_array_equal(qn["codes"], q["codes"] ^ 8)
    np.testing.assert_array_equal(qn["scales"], q["scales"])
    # the same permutation of a block's values and of H's rows and columns
    perm = rng.permutation(16)
    xp = x.reshape(8, 4, 16)[:, :, perm].reshape(8, 64)
    Hp = H[:, perm][:, :, perm]
    qp = Q.quantize_nvfp4_hessian(xp, Hp, 120)
    np.testing.assert_array_equal(qp["codes"].reshape(8, 4, 16), q["codes"].reshape(8, 4, 16)[:, :, perm])
    np.testing.assert_array_equal(qp["scales"], q["scales"])


def test_negative_control_transposed_blocks_fire():
    """Indexing H by the row's block number instead of its column block must
    fail the brute force (a plausible indexing mistake)."""
    rng = np.random.default_rng(80)
    x = _bf16(rng, (4, 64), heavy=True)
    H = synth.calibration_hessian(80, 0, 64, 96)
    q = Q.quantize_nvfp4_hessian(x, H, 96)
    S = _fr(q["tensor_scale"])
    wrong = 0
    for r in range(4):
        for b in range(4):
            c_wrong = _brute_block(x[r, 16 * b:16 * b + 16], H[r % 4], S)[0]
            wrong += c_wrong != q["scales"][r, b]
    assert wrong > 0
