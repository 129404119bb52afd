"""Pins of the oracle's UOS+EFQ mode (exp-free P~) against what the reading
fixes and what the mathematics implies.

The EFQ-Softmax page ("EFQ-Softmax", abstract) states the method's shape --
an exponent-only block scale from the local maximum, scores mapped to a
residual domain, nonnegative E2M1 codes by one affine rule, the same P~ in
numerator and denominator -- but prints none of its constants.  The reading
implemented (see oracle/mxoracle.c): code = clamp(rne(2 r + beta), 0, 7) on
the log2 residual r = z - e_b, beta fitted to the E2M1 rounding boundaries
of codes 2..7, e_b the smallest exponent keeping the block maximum below
code 8.  Parity of this mode with the pages themselves is unpinned (no
worked example or constant is printed); these tests pin the oracle to the
reading and to properties any such rule must have.
"""
import math

import numpy as np
import pytest

import oracle

MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# E2M1 round-to-nearest boundaries between codes c and c+1, c = 2..6, in log2
UPPER_BOUNDS = np.log2((MAG[2:7] + MAG[3:8]) / 2)


def code_boundaries():
    """Locations where oracle.efq_code steps up, found by bisection."""
    out = []
    r_lo = -3.0
    for target in range(1, 8):
        lo, hi = r_lo, 4.0
        assert oracle.efq_code(lo) < target <= oracle.efq_code(hi)
        for _ in range(80):
            mid = 0.5 * (lo + hi)
            if oracle.efq_code(mid) >= target:
                hi = mid
            else:
                lo = mid
        out.append(hi)
        r_lo = hi
    return np.array(out)


def test_code_rule_is_affine_two_codes_per_binade():
    b = code_boundaries()
    # seven unit steps, evenly spaced by half a binade (slope 2)
    assert np.allclose(np.diff(b), 0.5, atol=1e-12)
    assert [oracle.efq_code(x) for x in b + 1e-9] == list(range(1, 8))
    assert [oracle.efq_code(x) for x in b - 1e-9] == list(range(0, 7))


def test_code_rule_fits_the_e2m1_rounding_boundaries():
    b = code_boundaries()[2:7]  # boundaries between codes 2..7
    dev = b - UPPER_BOUNDS
    # least-squares fit of an evenly spaced grid: residuals sum to zero ...
    assert abs(dev.sum()) < 1e-9
    # ... and stay within the alternating 1.25/1.75 pattern's half-amplitude
    # (boundaries alternate 0.485 / 0.515 binades apart; three of one kind,
    # two of the other: deviations -0.0058 and +0.0087)
    assert np.abs(dev).max() < 0.009
    # the fitted offset is the one every boundary implies on average
    assert oracle.efq_beta() == pytest.approx(np.mean(np.arange(2, 7) + 0.5 - 2 * UPPER_BOUNDS), abs=1e-12)


def test_code_rule_clamps_and_ties_to_even():
    assert oracle.efq_code(-math.inf) == 0
    assert oracle.efq_code(-50.0) == 0
    assert oracle.efq_code(50.0) == 7
    beta = oracle.efq_beta()
    # exact ties of 2 r + beta at n + 1/2 round to the even code
    for n in range(0, 7):
        r = (n + 0.5 - beta) / 2
        if 2 * r + beta != n + 0.5:  # not exactly representable: skip
            continue
        assert oracle.efq_code(r) == (n if n % 2 == 0 else n + 1)


def test_block_exponent_is_the_smallest_that_keeps_the_max_below_code_8():
    rho = oracle.efq_rho()
    assert rho == pytest.approx((7.5 - oracle.efq_beta()) / 2 - 2.0 ** -10, abs=1e-15)
    rng = np.random.default_rng(3)
    for z in np.concatenate([-rng.exponential(8.0, 2000), [0.0, -1.0, -2.815, -300.0]]):
        e = oracle.efq_exponent(z)
        if z - (-127) >= rho:  # not clamped
            assert z - e < rho <= z - (e - 1)  # minimal
        else:
            assert e == -127
        if e > -127:
            # the block maximum gets one of the two top codes (5 only within
            # the 2^-10 margin below the 6 / 5 boundary)
            assert oracle.efq_code(z - e) in (5, 6, 7)
    assert oracle.efq_exponent(-math.inf) == -127
    # the row maximum itself (z = 0) is represented exactly: code 6 = 4 * 2^-2
    assert oracle.efq_exponent(0.0) == -2 and oracle.efq_code(2.0) == 6


def rand_qkv(seed, Sq=48, Skv=200, D=64, scale=1.5):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((1, 2, Sq, D)) * scale).astype(np.float32)
    k = (rng.standard_normal((1, 2, Skv, D)) * scale).astype(np.float32)
    v = rng.standard_normal((1, 2, Skv, D)).astype(np.float32)
    return q, k, v


def deq(x, rule):
    c, s = oracle.quantize(x, rule)
    return oracle.dequantize(c, s).reshape(x.shape)


def test_efq_pt_approximates_exp_within_the_rule_bound():
    """A code c >= 2 stands for a residual r with 2r + beta within 1/2 of c,
    and its magnitude is 2^((c - 2)/2) (times 1.5 / sqrt(2) for odd c), so
    log2(p~ / p) lies in [(beta - 2.5)/2, (beta - 1.5)/2 + log2(1.5) - 1/2]
    (about [-0.316, 0.269]); codes 0 and 1 only below the code-2 boundary."""
    q, k, v = rand_qkv(11)
    bc = 64
    rows = np.arange(2 * 48, dtype=np.int64)
    r = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_EFQ, bc=bc, rows=rows,
                         want_p=True, want_tiles=True)
    qt, kt = deq(q, oracle.RULE_UOS), deq(k, oracle.RULE_UOS)
    beta = oracle.efq_beta()
    for n in range(rows.size):
        h, i = divmod(n, 48)
        s = kt[0, h] @ qt[0, h, i] / 8.0
        codes = oracle.unpack_codes(r["p_codes"][n])[:200]
        scales = np.repeat(r["p_scales"][n].astype(np.int64), 32)[:200]
        for t in range(r["m_tiles"].shape[1]):
            sl = slice(t * bc, (t + 1) * bc)
            z = (s[sl] - r["m_tiles"][n, t]) / math.log(2.0)
            c, e = codes[sl] & 7, scales[sl] - 127
            assert not (codes[sl] & 8).any()  # nonnegative codes
            big = c >= 2
            dev = np.log2(MAG[c[big]]) + e[big] - z[big]
            assert dev.min() >= (beta - 2.5) / 2 - 1e-12
            assert dev.max() <= (beta - 1.5) / 2 + math.log2(1.5) - 0.5 + 1e-12
            small = c <= 1
            assert (z[small] - e[small] <= (1.5 - beta) / 2 + 1e-12).all()


def test_efq_v_ones_gives_one_and_equal_scores_give_the_mean():
    q, k, v = rand_qkv(12, Sq=16, Skv=150)
    rows = np.arange(32, dtype=np.int64)
    o = oracle.attn_rows(q, k, np.ones_like(v), causal=False, mode=oracle.MODE_UOS_EFQ, bc=64,
                         rows=rows)["o"]
    assert np.allclose(o, 1.0, atol=1e-14, rtol=0)
    # identical keys: every visible key gets the same code and scale, so O is
    # the plain mean of the quantized V over the keys
    k_same = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o = oracle.attn_rows(q, k_same, v, causal=False, mode=oracle.MODE_UOS_EFQ, bc=64, rows=rows)["o"]
    for n in range(32):
        h = n // 16
        c, s_ = oracle.quantize_t(v[0, h], oracle.RULE_UOS)
        vt = oracle.dequantize(c.reshape(-1), s_.reshape(-1)).reshape(64, -1).T[:150]
        assert np.allclose(o[n], vt.mean(axis=0), atol=1e-13, rtol=0)


def test_efq_denominator_is_sum_of_its_pt():
    q, k, v = rand_qkv(13, Sq=20, Skv=260)
    bc = 128
    rows = np.arange(40, dtype=np.int64)
    r = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_EFQ, bc=bc,
                         rows=rows, want_p=True, want_tiles=True)
    for n in range(40):
        vals = oracle.dequantize(r["p_codes"][n], r["p_scales"][n])
        w = np.empty_like(vals)
        for t in range(r["m_tiles"].shape[1]):
            w[t * bc:(t + 1) * bc] = math.exp(r["m_tiles"][n, t] - r["m"][n])
        assert r["l"][n] == pytest.approx(math.fsum(vals * w), rel=1e-13)


def test_efq_differs_from_exact_pnq_only_in_p():
    """Same Q~, K~, V~ and schedule: EFQ and UOS+PNQ outputs are close (the
    affine rule approximates exp-then-round), but not identical."""
    q, k, v = rand_qkv(14, Sq=32, Skv=256, scale=1.0)
    rows = np.arange(64, dtype=np.int64)
    a = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_EFQ, bc=128, rows=rows)["o"]
    b = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_PNQ, bc=128, rows=rows)["o"]
    assert not np.array_equal(a, b)
    assert np.abs(a - b).max() < 0.3 and np.abs(a - b).mean() < 0.05
