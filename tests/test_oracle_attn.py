"""Pins for the oracle's attention rows (CPU only).

The oracle is checked against: exact softmax attention (FP16 mode), the
closed-form cases the method fixes (q = 0, V = 1, a single visible key,
power-of-two rescaling of the operands, GQA = MHA with repeated K/V), the PNQ
statement that the denominator is the sum of the same quantized P~ that
feeds the numerator (MXAttention abstract; EFQ-Softmax abstract), and an
independent vectorised numpy recomputation of the P~ codes.
"""
import math

import numpy as np
import pytest

import mxsynth
import oracle

MODES = [oracle.MODE_OCP, oracle.MODE_UOS, oracle.MODE_UOS_PNQ]
RULE_OF = {oracle.MODE_OCP: oracle.RULE_OCP, oracle.MODE_UOS: oracle.RULE_UOS,
           oracle.MODE_UOS_PNQ: oracle.RULE_UOS}


def all_rows(B, H, S):
    return np.arange(B * H * S, dtype=np.int64)


def rand_qkv(seed, B=1, Hq=2, Hkv=2, Sq=100, Skv=100, D=64, scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, Sq, D)) * scale).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, Skv, D)) * scale).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    return q, k, v


def direct_softmax(q, k, v, causal):
    """Plain softmax(q k^T / sqrt(D)) v in binary64 (numpy)."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            s = q[b, h] @ k[b, h // g].T / math.sqrt(D)
            if causal:
                s = np.where(np.tril(np.ones_like(s, bool)), s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[b, h] = (p @ v[b, h // g]) / p.sum(axis=1, keepdims=True)
    return out


# Vectorised closed-form block quantizer, written independently of the C
# nearest search: exponent from frexp, codes by counting crossed boundaries
# (strict at boundaries whose lower neighbour has the even code, inclusive
# where the upper one has).
_STRICT = np.array([0.25, 1.25, 2.5, 5.0])
_INCL = np.array([0.75, 1.75, 3.5])
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def np_fake_quant_blocks(x, rule):
    """x [..., 32] binary64 -> (dequantized values, codes, E8M0 bytes)."""
    amax = np.abs(x).max(axis=-1)
    _, ex = np.frexp(amax)
    e = ex.astype(np.int64) - 3
    if rule == oracle.RULE_UOS:
        e = e + (amax > 7.25 * np.ldexp(1.0, e)).astype(np.int64)
    e = np.where(amax == 0, -127, np.clip(e, -127, 127))
    v = np.abs(x) * np.ldexp(1.0, -e)[..., None]
    code = (v[..., None] > _STRICT).sum(-1) + (v[..., None] >= _INCL).sum(-1)
    y = np.copysign(_MAG[code] * np.ldexp(1.0, e)[..., None], x)
    sign = np.signbit(x).astype(np.int64)
    return y, (sign << 3) | code, (e + 127).astype(np.int64)


def np_attn_row(qr, kt, vt, Skv, i, causal, mode, bc):
    """One row of the tiled online softmax in numpy (independent of C)."""
    rule = RULE_OF.get(mode)
    D = qr.size
    pad = (Skv + 31) // 32 * 32
    s_all = (kt[:Skv] @ qr) / math.sqrt(D)
    m, l, acc = -np.inf, 0.0, np.zeros(D)
    codes = np.zeros(pad, np.int64)
    scales = np.zeros(pad // 32, np.int64)
    for t0 in range(0, Skv, bc):
        hi = min(Skv, t0 + bc, i + 1 if causal else Skv)
        if hi <= t0:
            continue
        tl = min(t0 + bc, pad) - t0
        s = s_all[t0:hi]
        mnew = max(m, s.max())
        alpha = 0.0 if m == -np.inf else math.exp(m - mnew)
        p = np.zeros(tl)
        p[: hi - t0] = np.exp(s - mnew)
        if mode == oracle.MODE_FP16:
            pt = p
        else:
            pt, c, sc = np_fake_quant_blocks(p.reshape(-1, 32), rule)
            pt = pt.reshape(-1)
            codes[t0:t0 + tl] = c.reshape(-1)
            scales[t0 // 32:(t0 + tl) // 32] = sc
        l = alpha * l + (pt.sum() if mode == oracle.MODE_UOS_PNQ else p.sum())
        acc = alpha * acc + pt @ vt[t0:t0 + tl]
        m = mnew
    return acc / l, codes, scales


def deq_rows(x, rule):
    c, s = oracle.quantize(x, rule)
    return oracle.dequantize(c, s).reshape(x.shape)


def deq_keys(x2d, rule):
    """[S, D] -> dequantized, blocks along S, zero padded to 32: [S_pad, D]."""
    c, s = oracle.quantize_t(x2d, rule)
    D = x2d.shape[1]
    return oracle.dequantize(c.reshape(-1), s.reshape(-1)).reshape(D, -1).T


# --------------------------------------------------------------- FP16 mode --

def test_fp16_mode_equals_direct_softmax_tiny():
    q, k, v = mxsynth.tiny_attn(0)
    r = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_FP16, bc=128,
                         rows=all_rows(1, 1, 256))
    ref = direct_softmax(q, k, v, False).reshape(-1, 64)
    assert np.max(np.abs(r["o"] - ref)) < 1e-6
    assert np.max(np.abs(r["o"] - ref)) < 1e-12


def test_fp16_mode_equals_direct_softmax_causal_gqa_ragged():
    q, k, v = rand_qkv(1, B=2, Hq=4, Hkv=2, Sq=77, Skv=77, D=32)
    r = oracle.attn_rows(q, k, v, causal=True, mode=oracle.MODE_FP16, bc=32,
                         rows=all_rows(2, 4, 77))
    ref = direct_softmax(q, k, v, True).reshape(-1, 32)
    assert np.max(np.abs(r["o"] - ref)) < 1e-12


def test_fp16_mode_tile_invariance():
    q, k, v = rand_qkv(2, Sq=90, Skv=200)
    rows = all_rows(1, 2, 90)
    outs = [oracle.attn_rows(q, k, v, causal=False, mode=0, bc=bc, rows=rows)["o"]
            for bc in (32, 64, 128, 224)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-12


# ----------------------------------------------------- closed-form cases ----

@pytest.mark.parametrize("mode", MODES)
def test_q_zero_gives_mean_of_quantized_v(mode):
    q, k, v = rand_qkv(3, Sq=40, Skv=100)
    q[:] = 0
    r = oracle.attn_rows(q, k, v, causal=False, mode=mode, bc=64,
                         rows=all_rows(1, 2, 40), want_p=True)
    rule = RULE_OF[mode]
    for h in range(2):
        vt = deq_keys(v[0, h], rule)[:100]
        assert np.allclose(r["o"][h * 40:(h + 1) * 40], vt.mean(axis=0)[None], atol=1e-14, rtol=0)
    # every visible p is exactly 1 -> code 6 (4.0) under scale 2^-2
    codes = oracle.unpack_codes(r["p_codes"])
    assert np.all(codes[:, :100] == 6) and np.all(codes[:, 100:] == 0)
    assert np.all(r["p_scales"][:, :3] == 125)
    # last block holds keys 96..99 (max 1) and zero padding
    assert np.all(r["p_scales"][:, 3] == 125)


@pytest.mark.parametrize("mode", MODES)
def test_v_ones(mode):
    """V = 1 is exact in MXFP4 (4 * 2^-2).  Under PNQ numerator and
    denominator sum the same P~, so O = 1 by construction; the non-PNQ modes
    divide sum(P~) by sum(P) and miss 1."""
    q, k, v = rand_qkv(4, Sq=50, Skv=150, scale=2.0)
    v[:] = 1.0
    o = oracle.attn_rows(q, k, v, causal=False, mode=mode, bc=64, rows=all_rows(1, 2, 50))["o"]
    if mode == oracle.MODE_UOS_PNQ:
        assert np.max(np.abs(o - 1.0)) < 1e-14
    else:
        assert np.max(np.abs(o - 1.0)) > 1e-3


@pytest.mark.parametrize("mode", [0] + MODES)
def test_causal_first_row_is_first_value(mode):
    q, k, v = rand_qkv(5, Sq=64, Skv=64)
    rows = np.array([0, 64], np.int64)  # row 0 of heads 0 and 1
    o = oracle.attn_rows(q, k, v, causal=True, mode=mode, bc=32, rows=rows)["o"]
    for j, h in enumerate((0, 1)):
        v0 = v[0, h, 0].astype(np.float64) if mode == 0 else deq_keys(v[0, h], RULE_OF[mode])[0]
        assert np.array_equal(o[j], v0)


@pytest.mark.parametrize("mode", [0] + MODES)
def test_power_of_two_rescaling(mode):
    """Q * 2^-k with K * 2^k leaves O unchanged; V * 2^k scales O by 2^k
    (exact power-of-two scales, 'Quantization Error')."""
    q, k, v = rand_qkv(6, Sq=33, Skv=97)
    rows = all_rows(1, 2, 33)
    base = oracle.attn_rows(q, k, v, causal=False, mode=mode, bc=64, rows=rows)["o"]
    for kk in (-3, 5):
        f = np.float32(2.0 ** kk)
        o1 = oracle.attn_rows(q / f, k * f, v, causal=False, mode=mode, bc=64, rows=rows)["o"]
        assert np.array_equal(o1, base)
        o2 = oracle.attn_rows(q, k, v * f, causal=False, mode=mode, bc=64, rows=rows)["o"]
        assert np.array_equal(o2, base * float(f))


@pytest.mark.parametrize("mode", [0] + MODES)
def test_gqa_equals_mha_with_repeated_kv(mode):
    q, k, v = rand_qkv(7, B=2, Hq=6, Hkv=2, Sq=45, Skv=45, D=32)
    rows = all_rows(2, 6, 45)
    o = oracle.attn_rows(q, k, v, causal=True, mode=mode, bc=32, rows=rows)["o"]
    k3 = np.repeat(k, 3, axis=1)
    v3 = np.repeat(v, 3, axis=1)
    o3 = oracle.attn_rows(q, k3, v3, causal=True, mode=mode, bc=32, rows=rows)["o"]
    assert np.array_equal(o, o3)


# ------------------------------------------------------------------ PNQ ----

def _weighted_pt(r, Skv, bc):
    """Dequantized P~ of each dumped row, each tile's block weighted by
    exp(m_tile - m_final)."""
    out = []
    for n in range(r["p_codes"].shape[0]):
        vals = oracle.dequantize(r["p_codes"][n], r["p_scales"][n])
        w = np.empty_like(vals)
        for t in range(r["m_tiles"].shape[1]):
            mt = r["m_tiles"][n, t]
            w[t * bc:(t + 1) * bc] = 0.0 if mt == -np.inf else math.exp(mt - r["m"][n])
        out.append(vals * w)
    return out


def test_pnq_denominator_is_sum_of_quantized_p():
    q, k, v = rand_qkv(8, Sq=60, Skv=300, scale=1.5)
    bc = 64
    r = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_PNQ, bc=bc,
                         rows=all_rows(1, 2, 60), want_p=True, want_tiles=True)
    for n, wp in enumerate(_weighted_pt(r, 300, bc)):
        assert r["l"][n] == pytest.approx(math.fsum(wp), rel=1e-13)
        h = n // 60
        vt = deq_keys(v[0, h], oracle.RULE_UOS)
        assert np.allclose(r["o"][n], (wp @ vt) / math.fsum(wp), atol=1e-13, rtol=0)


def test_non_pnq_denominator_is_sum_of_unquantized_p():
    q, k, v = rand_qkv(9, Sq=20, Skv=130)
    r = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS, bc=32,
                         rows=all_rows(1, 2, 20), want_p=True)
    qt = deq_rows(q, oracle.RULE_UOS)
    kt = deq_rows(k, oracle.RULE_UOS)
    for n in range(40):
        h, i = divmod(n, 20)
        s = kt[0, h] @ qt[0, h, i] / 8.0
        assert r["l"][n] == pytest.approx(np.exp(s - s.max()).sum(), rel=1e-13)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True])
def test_independent_recomputation(mode, causal):
    """P~ codes, E8M0 bytes and O against the numpy recomputation."""
    q, k, v = rand_qkv(10 + mode, B=1, Hq=2, Hkv=1, Sq=130, Skv=130, D=64, scale=1.7)
    bc = 64
    rows = all_rows(1, 2, 130)
    r = oracle.attn_rows(q, k, v, causal=causal, mode=mode, bc=bc, rows=rows, want_p=True)
    rule = RULE_OF[mode]
    qt = deq_rows(q, rule)
    kt = deq_rows(k, rule)
    vt = deq_keys(v[0, 0], rule)
    for n in range(rows.size):
        h, i = divmod(n, 130)
        o, codes, scales = np_attn_row(qt[0, h, i], kt[0, 0], vt, 130, i, causal, mode, bc)
        assert np.allclose(r["o"][n], o, atol=1e-12, rtol=0)
        assert np.array_equal(oracle.unpack_codes(r["p_codes"][n]), codes)
        assert np.array_equal(r["p_scales"][n], scales)


def test_fp16_independent_recomputation_mode_schedule():
    q, k, v = rand_qkv(20, Sq=30, Skv=170)
    r = oracle.attn_rows(q, k, v, causal=False, mode=0, bc=96, rows=all_rows(1, 2, 30))
    for n in range(60):
        h, i = divmod(n, 30)
        o, _, _ = np_attn_row(q[0, h, i].astype(np.float64), k[0, h].astype(np.float64),
                              np.r_[v[0, h].astype(np.float64), np.zeros((22, 64))],
                              170, i, False, 0, 96)
        assert np.allclose(r["o"][n], o, atol=1e-13, rtol=0)


def test_quantized_modes_depend_on_tile_schedule():
    """P~ depends on the running max at each tile: different Bc give
    (slightly) different O in the quantized modes."""
    q, k, v = rand_qkv(21, Sq=16, Skv=512, scale=1.5)
    rows = all_rows(1, 2, 16)
    a = oracle.attn_rows(q, k, v, causal=False, mode=3, bc=32, rows=rows)["o"]
    b = oracle.attn_rows(q, k, v, causal=False, mode=3, bc=512, rows=rows)["o"]
    assert not np.array_equal(a, b)
    assert np.max(np.abs(a - b)) < 0.2


def test_bad_arguments_rejected():
    q, k, v = rand_qkv(0, Sq=8, Skv=8, D=32)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, k, v, causal=False, mode=1, bc=48, rows=[0])
    with pytest.raises(ValueError):
        oracle.attn_rows(q, k, v, causal=False, mode=7, bc=64, rows=[0])
    with pytest.raises(ValueError):
        oracle.attn_rows(q, k, v, causal=False, mode=1, bc=64, rows=[10 ** 6])
