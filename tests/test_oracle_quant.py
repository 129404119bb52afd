"""Pins for the oracle's block quantizer (CPU only).

Each test checks the oracle against something other than itself: the E2M1
table of the OCP MX specification, the worked error figures of the
"Quantization Error" page, an exact-rational nearest search, the closed form
of the scale exponent, the MSE argument that fixes 7.25, and the exact
power-of-two properties stated on the "Quantization Error" page.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import mxsynth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


E2M1 = {int(c): float(v) for c, v in _read_golden("e2m1_codes.txt")}
MAGS = [Fraction(E2M1[c]) for c in range(8)]
QMAX = float(dict(_read_golden("uos_boundary.txt"))["qmax"])


def ref_code(v: Fraction) -> int:
    """Exact-rational nearest E2M1 magnitude; ties go to the even code."""
    best = None
    for c, g in enumerate(MAGS):
        d = abs(v - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def closed_form_exponent(amax: float, rule: int) -> int:
    """Scale exponent from frexp: E = floor(log2 amax); OCP e = E - 2;
    UOS moves one up when amax / 2^(E-2) exceeds 7.25; clamp to E8M0."""
    if amax == 0.0:
        return -127
    m, ex = math.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1)
    E = ex - 1
    e = E - 2
    if rule == oracle.RULE_UOS and Fraction(amax) > Fraction(QMAX) * Fraction(2) ** e:
        e += 1
    return max(-127, min(127, e))


def ref_quantize_block(x, rule):
    amax = max(abs(float(t)) for t in x)
    e = closed_form_exponent(amax, rule)
    codes = []
    for t in x:
        v = abs(Fraction(float(t))) / Fraction(2) ** e
        codes.append((8 if math.copysign(1.0, float(t)) < 0 else 0) | ref_code(v))
    return e + 127, codes


# ---------------------------------------------------------------- grid ----

def test_decode_matches_spec_table():
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    for X in (0, 100, 127, 130, 254):
        y = oracle.dequantize(np.tile(packed, 4), np.full(2, X, np.uint8))[:16]
        for c in range(16):
            want = E2M1[c] * 2.0 ** (X - 127)
            assert y[c] == want and math.copysign(1, y[c]) == math.copysign(1, want)


def test_grid_members_are_fixed_points():
    for c in range(8):
        assert oracle.round_e2m1(E2M1[c]) == c


def test_round_exhaustive_bf16():
    """Every finite non-negative bf16 value against the rational search."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    vals = mxsynth.bf16_bits_to_f32(bits).astype(np.float64)
    for v in vals:
        assert oracle.round_e2m1(float(v)) == ref_code(Fraction(float(v))), v


def test_round_dense_fp32_around_every_boundary():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for b in mids:
        x = np.float32(b)
        lo = x
        for _ in range(64):
            lo = np.nextafter(lo, np.float32(0))
        v = lo
        for _ in range(129):
            assert oracle.round_e2m1(float(v)) == ref_code(Fraction(float(v))), float(v)
            v = np.nextafter(v, np.float32(np.inf))
    rng = np.random.default_rng(11)
    for v in rng.uniform(0, 9, 20000).astype(np.float32):
        assert oracle.round_e2m1(float(v)) == ref_code(Fraction(float(v)))


def test_ties_go_to_even_code():
    # (tie value, expected code): 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0,
    # 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0
    for v, c in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]:
        assert oracle.round_e2m1(v) == c


def test_worst_case_error_worked_on_page():
    for v, r, err in _read_golden("qe_worst_case.txt"):
        v, r, err = float(v), float(r), float(err)
        got = E2M1[oracle.round_e2m1(v)]
        assert got == r
        assert abs(v - got) / v == pytest.approx(err, abs=1e-15)


def test_saturation():
    for v in (6.0, 6.5, 7.25, 7.99, 8.0, 1e30):
        assert oracle.round_e2m1(v) == 7


# ---------------------------------------------------------- scale rule ----

def _amax_cases():
    out = [0.0, 5e-324, 2.0 ** -149, 2.0 ** -130, 2.0 ** -127, 2.0 ** -126,
           float(np.finfo(np.float32).max)]
    for k in range(-140, 125, 7):
        for base in (1.0, 1.5, 1.8125, 3.625, 7.25, 8.0):
            a = base * 2.0 ** k
            out += [a, np.nextafter(a, np.inf), np.nextafter(a, 0.0)]
    return [float(a) for a in out if a < 3.4e38]


@pytest.mark.parametrize("rule", [oracle.RULE_OCP, oracle.RULE_UOS])
def test_scale_exponent_closed_form(rule):
    for a in _amax_cases():
        assert oracle.scale_exponent(a, rule) == closed_form_exponent(a, rule), a


def test_uos_boundary_is_inclusive_and_exact():
    for k in range(-100, 100, 3):
        a = QMAX * 2.0 ** k
        assert oracle.scale_exponent(a, oracle.RULE_UOS) == k
        assert oracle.scale_exponent(np.nextafter(a, np.inf), oracle.RULE_UOS) == k + 1
        # OCP puts the same amax in [4, 8)
        assert oracle.scale_exponent(a, oracle.RULE_OCP) == k


def test_scaled_amax_ranges_bruteforce_bf16():
    """Over every positive normal bf16 amax: OCP leaves amax/2^e in [4, 8),
    UOS in (3.625, 7.25]; UOS differs from OCP exactly when the OCP ratio
    exceeds 7.25, and then by one exponent."""
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint16)
    vals = mxsynth.bf16_bits_to_f32(bits).astype(np.float64)
    for a in vals[::3]:
        eo = oracle.scale_exponent(a, oracle.RULE_OCP)
        eu = oracle.scale_exponent(a, oracle.RULE_UOS)
        ro = a / 2.0 ** eo
        ru = a / 2.0 ** eu
        if eo > -127:
            assert 4.0 <= ro < 8.0
            assert 3.625 < ru <= 7.25
        assert eu - eo == (1 if ro > 7.25 else 0)


def test_amax_element_clipping_error_bounds():
    """Relative error of a block maximum that saturates (scaled amax > 6):
    OCP's supremum is 25% (never reached), UOS's maximum is 1.25/7.25; and
    without clipping no element errs by more than the page's 20%."""
    rng = np.random.default_rng(5)
    worst_clip = {0: 0.0, 1: 0.0}
    worst_any = 0.0
    for a in np.concatenate([rng.uniform(1, 2, 4000), [1.8125, 1.8125 + 1e-12, 1.999999]]):
        for rule in (0, 1):
            e = oracle.scale_exponent(a, rule)
            r = a / 2.0 ** e
            q = E2M1[oracle.round_e2m1(r)] * 2.0 ** e
            err = abs(a - q) / a
            if r > 6.0:
                worst_clip[rule] = max(worst_clip[rule], err)
            else:
                worst_any = max(worst_any, err)
    assert 0.24 < worst_clip[0] < 0.25
    assert worst_clip[1] == pytest.approx(1.25 / 7.25, rel=1e-9)
    assert worst_any <= 0.2 + 1e-15


def _mse_uniform(r, scale_mult, n=200001):
    """Mean squared error (in units of s^2) of quantizing values uniform on
    [0, r*s] at scale scale_mult*s, by midpoint quadrature through the
    oracle's element rounding."""
    xs = (np.arange(n) + 0.5) / n * r
    v = xs / scale_mult
    codes = np.fromiter((oracle.round_e2m1(float(t)) for t in v), np.int64, n)
    q = np.array([E2M1[c] for c in range(8)])[codes] * scale_mult
    return float(np.mean((xs - q) ** 2))


def test_qmax_is_the_uniform_mse_crossover():
    """For elements uniform in [0, amax], keeping scale s or moving to 2s
    costs the same squared error exactly at amax/s = 7.25: below it the
    smaller scale wins, above it the larger one.  This fixes the constant
    and the direction of the UOS rule independently of its code."""
    below = _mse_uniform(7.2, 1.0) - _mse_uniform(7.2, 2.0)
    above = _mse_uniform(7.3, 1.0) - _mse_uniform(7.3, 2.0)
    at = _mse_uniform(7.25, 1.0) - _mse_uniform(7.25, 2.0)
    assert below < -1e-3 and above > 1e-3
    assert abs(at) < 2e-4
    # closed form of the two error integrals: 7/8 + (r-6)^3/3 vs 5/3 - (8-r)^3/3
    for r in (7.2, 7.25, 7.3):
        assert _mse_uniform(r, 1.0) == pytest.approx((7 / 8 + (r - 6) ** 3 / 3) / r, rel=1e-6)
        assert _mse_uniform(r, 2.0) == pytest.approx((5 / 3 - (8 - r) ** 3 / 3) / r, rel=1e-6)
    # and the UOS rule switches exactly there
    assert oracle.scale_exponent(7.25, oracle.RULE_UOS) == 0
    assert oracle.scale_exponent(7.2500001, oracle.RULE_UOS) == 1


# --------------------------------------------------------------- blocks ----

@pytest.mark.parametrize("rule", [oracle.RULE_OCP, oracle.RULE_UOS])
def test_blocks_match_rational_reference(rule):
    x = mxsynth.tiny_quant(1)
    sel = np.r_[0:160, 2048:2208, 4000:4096]
    codes, scales = oracle.quantize(x, rule)
    cu = oracle.unpack_codes(codes.reshape(-1, 16))
    for b in sel:
        X, c = ref_quantize_block(x[b], rule)
        assert scales[b] == X
        assert list(cu[b]) == c


def test_edge_blocks():
    f32 = np.float32
    blocks = [
        np.zeros(32, f32),
        -np.zeros(32, f32),
        np.r_[f32(7.25), np.zeros(31, f32)],
        np.r_[f32(-1e-40), np.full(31, f32(1e-45))],  # fp32 subnormals
        np.full(32, np.finfo(f32).max),
        np.r_[f32(1.0), np.full(31, f32(-0.001))],    # negatives rounding to -0
        np.linspace(-6, 6, 32).astype(f32),
    ]
    for rule in (0, 1):
        for blk in blocks:
            codes, scales = oracle.quantize(blk, rule)
            X, c = ref_quantize_block(blk, rule)
            assert scales[0] == X
            assert list(oracle.unpack_codes(codes)) == c
    # zero block: X = 0, codes 0; negative zeros keep their sign bit
    c, s = oracle.quantize(-np.zeros(32, f32), 1)
    assert s[0] == 0 and np.all(c == 0x88)


@pytest.mark.parametrize("rule", [oracle.RULE_OCP, oracle.RULE_UOS])
def test_scale_periodicity(rule):
    """x * 2^k quantizes to the same codes with the E8M0 byte shifted by k
    (the scale applies exactly)."""
    x = mxsynth.tiny_quant(1)
    c0, s0 = oracle.quantize(x, rule)
    for k in (-40, -7, -1, 1, 3, 29):
        c1, s1 = oracle.quantize((x * np.float32(2.0 ** k)).astype(np.float32), rule)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_block_order_independence():
    x = mxsynth.tiny_quant(1)
    perm = np.random.default_rng(3).permutation(x.shape[0])
    c0, s0 = oracle.quantize(x, 1)
    c1, s1 = oracle.quantize(x[perm], 1)
    assert np.array_equal(c1.reshape(-1, 16), c0.reshape(-1, 16)[perm])
    assert np.array_equal(s1, s0[perm])


def test_transposed_matches_flat_on_transpose():
    rng = np.random.default_rng(9)
    for rows in (32, 64, 57, 1, 33):
        x = rng.standard_normal((rows, 48)).astype(np.float32)
        ct, st = oracle.quantize_t(x, 1)
        rp = (rows + 31) // 32 * 32
        xp = np.zeros((rp, 48), np.float32)
        xp[:rows] = x
        cf, sf = oracle.quantize(np.ascontiguousarray(xp.T), 1)
        assert np.array_equal(ct.reshape(-1), cf)
        assert np.array_equal(st.reshape(-1), sf)


def test_bf16_input_path_equals_fp32_path():
    x = mxsynth.tiny_quant(1)
    xb = mxsynth.f32_to_bf16_bits(x)
    xw = mxsynth.bf16_bits_to_f32(xb)
    assert np.array_equal(oracle.quantize(xb, 1)[0], oracle.quantize(xw, 1)[0])
    assert np.array_equal(oracle.quantize(xb, 1)[1], oracle.quantize(xw, 1)[1])


def test_relative_frobenius_error_sane():
    """Round trip of Gaussian blocks: relative Frobenius error well under the
    0.10 'look at this layer' level of the 'Quantization Error' page, UOS at
    or below OCP."""
    x = mxsynth.tiny_quant(1)[:2048]
    errs = {}
    for rule in (0, 1):
        c, s = oracle.quantize(x, rule)
        y = oracle.dequantize(c, s)
        errs[rule] = np.linalg.norm(x.reshape(-1) - y) / np.linalg.norm(x)
    assert 0.05 < errs[1] <= errs[0] < 0.2
