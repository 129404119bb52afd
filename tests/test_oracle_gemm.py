"""Pins of the oracle's W4A4 product (``oracle.gemm_q`` / ``oracle.gemm``).

The product of two MXFP4 operands quantized along the contraction
("MXCode", abstract: MX-native W4A4 operands) is a plain definition:
y[m, n] = sum_k deq(a)[m, k] deq(b)[n, k].  The pins tie the oracle to it
without going through the oracle's own decode: an exact rational sum built
from the E2M1 table of the OCP specification (``tests/golden/e2m1_codes.txt``),
operands already on the grid (quantization is the identity and the product
is exact in binary64), power-of-two scaling, and invariance under a common
permutation of the 32-blocks of K ("Quantization Error", section "Where the
error comes from": each block carries its own exact power-of-two scale, so
block order does not matter).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e2m1_codes.txt")


def e2m1_table():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        vals[int(c)] = Fraction(v)
    assert sorted(vals) == list(range(16))
    return vals


def exact_values(codes, scales, rows, K):
    """Fractions of a [rows, K] operand decoded straight from the bytes."""
    tab = e2m1_table()
    codes = codes.reshape(rows, K // 2)
    scales = scales.reshape(rows, K // 32)
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            byte = int(codes[r, k // 2])
            c = byte & 0xF if k % 2 == 0 else byte >> 4
            row.append(tab[c] * Fraction(2) ** (int(scales[r, k // 32]) - 127))
        out.append(row)
    return out


@pytest.mark.parametrize("rule", [oracle.RULE_OCP, oracle.RULE_UOS])
def test_gemm_matches_exact_rational_sum(rule):
    rng = np.random.default_rng(40 + rule)
    M, N, K = 5, 4, 96
    a = (rng.standard_t(3, (M, K)) * 0.3).astype(np.float32)
    b = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-6, 6, (N, 1)))).astype(np.float32)
    y, yabs, (ac, as_), (bc, bs) = oracle.gemm(a, b, rule)
    A = exact_values(ac, as_, M, K)
    B = exact_values(bc, bs, N, K)
    for m in range(M):
        for n in range(N):
            exact = sum(A[m][k] * B[n][k] for k in range(K))
            absum = sum(abs(A[m][k] * B[n][k]) for k in range(K))
            # binary64 summation of K exact products
            assert abs(Fraction(y[m, n]) - exact) <= 2 * K * Fraction(2) ** -53 * absum
            assert abs(Fraction(yabs[m, n]) - absum) <= 2 * K * Fraction(2) ** -53 * absum


def on_grid(rng, rows, K, emin=-3, emax=3):
    """Blocks of E2M1 values times 2^e, each with one element at +-6 * 2^e,
    so that both scale rules reproduce them exactly."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = mags[rng.integers(0, 8, (rows, K))] * rng.choice([-1.0, 1.0], (rows, K))
    x = x.reshape(rows, K // 32, 32)
    x[:, :, 0] = 6.0 * rng.choice([-1.0, 1.0], (rows, K // 32))
    e = rng.integers(emin, emax + 1, (rows, K // 32, 1)).astype(np.float64)
    return (x * np.exp2(e)).reshape(rows, K).astype(np.float32)


@pytest.mark.parametrize("rule", [oracle.RULE_OCP, oracle.RULE_UOS])
def test_on_grid_operands_give_the_exact_product(rule):
    rng = np.random.default_rng(50 + rule)
    M, N, K = 33, 17, 512
    a, b = on_grid(rng, M, K), on_grid(rng, N, K)
    y, yabs, (ac, as_), _ = oracle.gemm(a, b, rule)
    # the quantizer reproduces the operand ...
    assert np.array_equal(oracle.dequantize(ac, as_).reshape(M, K), a.astype(np.float64))
    # ... and every partial sum is a multiple of 2^-8 below 2^21: exact
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.array_equal(y, ref)
    assert np.array_equal(yabs, np.abs(a.astype(np.float64)) @ np.abs(b.astype(np.float64)).T)


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(60)
    M, N, K = 12, 9, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    y0 = oracle.gemm(a, b, oracle.RULE_UOS)[0]
    for k in (-20, -3, 5, 40):
        yk = oracle.gemm(a * np.float32(2.0 ** k), b, oracle.RULE_UOS)[0]
        assert np.array_equal(yk, y0 * 2.0 ** k)


def test_block_permutation_invariance():
    rng = np.random.default_rng(61)
    M, N, K = 10, 7, 384
    a = rng.standard_t(3, (M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    perm = rng.permutation(K // 32)
    pa = a.reshape(M, K // 32, 32)[:, perm].reshape(M, K)
    pb = b.reshape(N, K // 32, 32)[:, perm].reshape(N, K)
    y, yabs = oracle.gemm(a, b, oracle.RULE_UOS)[:2]
    yp = oracle.gemm(pa, pb, oracle.RULE_UOS)[0]
    assert np.all(np.abs(yp - y) <= 2 * K * 2.0 ** -53 * yabs)


def test_row_subset_and_chunking_agree():
    rng = np.random.default_rng(62)
    M, N, K = 40, 50, 128
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    y, _, qa, qb = oracle.gemm(a, b, oracle.RULE_OCP)
    rows = np.array([39, 0, 17])
    ys, ysabs = oracle.gemm_q(qa[0], qa[1], qb[0], qb[1], M, N, K, rows=rows, n_chunk=7)
    assert np.all(np.abs(ys - y[rows]) <= 2 * K * 2.0 ** -53 * ysabs)
