"""Pins for the oracle's split-key attention and end-aligned causal queries
(the short-query, long-key case): keys cut into splits that each run the
tiled online softmax on their own ("EFQ-Softmax", abstract: running-max
update, history rescaling and final normalization as in FlashAttention),
merged in order by rescaling.

Checked against: exact softmax (FP16 mode, any split), an independent numpy
recomputation of the split schedule (P~ codes, E8M0 bytes and O in the
quantized modes), the unsplit oracle when one split covers every key, the
PNQ identity V = 1 -> O = 1, and the last query row of an end-aligned causal
block, which sees every key.
"""
import math

import numpy as np
import pytest

import oracle
from test_oracle_attn import (RULE_OF, deq_keys, deq_rows, np_fake_quant_blocks,
                              rand_qkv)

MODES = [oracle.MODE_OCP, oracle.MODE_UOS, oracle.MODE_UOS_PNQ]


def direct_softmax_end_causal(q, k, v, causal):
    """softmax(q k^T / sqrt(D)) v in binary64; causal query i sees keys
    j <= i + Skv - Sq."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            s = q[b, h] @ k[b, h // g].T / math.sqrt(D)
            if causal:
                vis = np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + (Skv - Sq)
                s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[b, h] = (p @ v[b, h // g]) / p.sum(axis=1, keepdims=True)
    return out


def np_split_row(qr, kt, vt, Skv, klim, mode, bc, split):
    """One query row, split schedule, in numpy (independent of the C code):
    each split runs its tiles from m = -inf; splits merge in order."""
    rule = RULE_OF.get(mode)
    D = qr.size
    pad = (Skv + 31) // 32 * 32
    s_all = (kt[:Skv] @ qr) / math.sqrt(D)
    codes = np.zeros(pad, np.int64)
    scales = np.zeros(pad // 32, np.int64)
    M, L, A = -np.inf, 0.0, np.zeros(D)
    split = split or ((Skv + bc - 1) // bc) * bc
    for s0 in range(0, Skv, split):
        m, l, acc = -np.inf, 0.0, np.zeros(D)
        for t0 in range(s0, min(s0 + split, Skv), bc):
            hi = min(Skv, t0 + bc, klim + 1)
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
        if m == -np.inf:
            continue
        Mn = max(M, m)
        wa = 0.0 if M == -np.inf else math.exp(M - Mn)
        wb = math.exp(m - Mn)
        A, L, M = A * wa + acc * wb, L * wa + l * wb, Mn
    return A / L, codes, scales


@pytest.mark.parametrize("split", [64, 128, 192])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_split_equals_direct_softmax(split, causal):
    q, k, v = rand_qkv(30, B=2, Hq=4, Hkv=2, Sq=5, Skv=300, D=64, scale=1.5)
    rows = np.arange(2 * 4 * 5, dtype=np.int64)
    r = oracle.attn_rows(q, k, v, causal=causal, mode=oracle.MODE_FP16, bc=64, rows=rows,
                         split=split)
    ref = direct_softmax_end_causal(q, k, v, causal).reshape(-1, 64)
    assert np.allclose(r["o"], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(7, 300, 64), (4, 257, 64)])
def test_split_independent_recomputation(mode, causal, shape):
    """P~ codes, E8M0 bytes and O of the split schedule against numpy.
    (Sq=4, Skv=257, split 64: the last split holds key 256 only, which the
    causal rows 0..2 do not see -- a split with no visible key.)"""
    Sq, Skv, split = shape
    q, k, v = rand_qkv(31 + mode, B=1, Hq=2, Hkv=1, Sq=Sq, Skv=Skv, D=64, scale=1.6)
    bc = 64
    rows = np.arange(2 * Sq, dtype=np.int64)
    r = oracle.attn_rows(q, k, v, causal=causal, mode=mode, bc=bc, rows=rows, want_p=True,
                         split=split)
    rule = RULE_OF[mode]
    qt, kt, vt = deq_rows(q, rule), deq_rows(k, rule), deq_keys(v[0, 0], rule)
    for n in range(rows.size):
        h, i = divmod(n, Sq)
        klim = i + Skv - Sq if causal else Skv - 1
        o, codes, scales = np_split_row(qt[0, h, i], kt[0, 0], vt, Skv, klim, mode, bc, split)
        assert np.allclose(r["o"][n], o, atol=1e-12, rtol=0)
        assert np.array_equal(oracle.unpack_codes(r["p_codes"][n]), codes)
        assert np.array_equal(r["p_scales"][n], scales)


@pytest.mark.parametrize("mode", [oracle.MODE_FP16] + MODES + [oracle.MODE_UOS_EFQ])
def test_one_split_covering_all_keys_is_the_unsplit_result(mode):
    q, k, v = rand_qkv(32, B=1, Hq=2, Hkv=2, Sq=9, Skv=300, D=64, scale=1.4)
    rows = np.arange(18, dtype=np.int64)
    a = oracle.attn_rows(q, k, v, causal=False, mode=mode, bc=64, rows=rows, want_p=True)
    b = oracle.attn_rows(q, k, v, causal=False, mode=mode, bc=64, rows=rows, want_p=True,
                         split=320)
    for key in ("o", "l", "m"):
        assert np.array_equal(a[key], b[key])
    if mode != oracle.MODE_FP16:
        assert np.array_equal(a["p_codes"], b["p_codes"])


@pytest.mark.parametrize("mode", [oracle.MODE_UOS_PNQ, oracle.MODE_UOS_EFQ])
def test_split_v_ones_gives_one(mode):
    q, k, v = rand_qkv(33, B=1, Hq=2, Hkv=1, Sq=6, Skv=500, D=64, scale=2.0)
    r = oracle.attn_rows(q, k, np.ones_like(v), causal=True, mode=mode, bc=64,
                         rows=np.arange(12, dtype=np.int64), split=128)
    assert np.allclose(r["o"], 1.0, atol=1e-14, rtol=0)


def test_split_changes_quantized_p_but_not_much():
    """Each split scales its P~ blocks by its own running max, so splits
    change O slightly in the quantized modes (and not at all in FP16 mode,
    where the merge is exact)."""
    q, k, v = rand_qkv(34, B=1, Hq=2, Hkv=2, Sq=8, Skv=1024, D=64, scale=1.5)
    rows = np.arange(16, dtype=np.int64)
    a = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_PNQ, bc=128, rows=rows)
    b = oracle.attn_rows(q, k, v, causal=False, mode=oracle.MODE_UOS_PNQ, bc=128, rows=rows,
                         split=256)
    assert not np.array_equal(a["o"], b["o"])
    assert np.abs(a["o"] - b["o"]).max() < 0.2


def test_end_aligned_causal_last_row_sees_every_key():
    q, k, v = rand_qkv(35, B=1, Hq=2, Hkv=1, Sq=3, Skv=200, D=64)
    rows = np.array([2, 5], dtype=np.int64)  # i = Sq - 1 of both heads
    for mode in (oracle.MODE_FP16, oracle.MODE_UOS_PNQ):
        a = oracle.attn_rows(q, k, v, causal=True, mode=mode, bc=64, rows=rows, split=128)
        b = oracle.attn_rows(q, k, v, causal=False, mode=mode, bc=64, rows=rows, split=128)
        assert np.array_equal(a["o"], b["o"])


def test_split_arguments_checked():
    q, k, v = rand_qkv(36, Sq=4, Skv=100, D=32)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, k, v, causal=False, mode=1, bc=64, rows=[0], split=96)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, k[:, :, :3], v[:, :, :3], causal=True, mode=1, bc=64, rows=[0])
