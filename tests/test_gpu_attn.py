"""GPU parity of MXFP4 attention (all modes) against the binary64 oracle.

Checked per case: the quantized K~ and V~^T that the prepare step leaves in
the workspace, and the Q~ that the kernel forms in its prologue (stored by
the dump variant), are bit-exact; O matches within max-abs 2e-3 and mean-abs 2e-4; the fraction
of P~ elements that differ from the oracle (read back through the dump
entry point) is at most 1e-4; the dump variant returns the same O bits as
the plain entry point.
"""
import functools

import numpy as np
import pytest

from common import (FLIP_MAX, MAX_ABS, MEAN_ABS, MODE_IDS, RULE_IDS, RULE_OF_MODE,
                    decode_kv_images, flips, gpu, mxsynth, np_u8, oracle, to_torch)

pytestmark = pytest.mark.gpu

ALL_MODES = ["fp16", "ocp", "uos", "uos_pnq", "uos_efq"]
MX_MODES = ["ocp", "uos", "uos_pnq", "uos_efq"]


def check_workspace(mx, ws, q, k, v, mode, with_q):
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    off, skv_ld = mx.workspace_layout(B, Hq, Hkv, Sq, Skv, D,
                                      "bf16" if q.dtype == np.uint16 else "f32", mode)
    w = np_u8(ws)
    rule = RULE_IDS[RULE_OF_MODE[mode]]
    if with_q:
        rc, rs = oracle.quantize(q, rule)
        assert np.array_equal(w[off[0]:off[0] + rc.size], rc)
        assert np.array_equal(w[off[1]:off[1] + rs.size], rs)
    kc, ks, vc, vs, pad = decode_kv_images(w, off, B, Hkv, Skv, D)
    assert skv_ld == kc.shape[1]
    assert not pad.any()
    pad32 = (Skv + 31) // 32 * 32
    for bg in range(B * Hkv):
        rc, rs = oracle.quantize(k.reshape(B * Hkv, Skv, D)[bg], rule)
        assert np.array_equal(kc[bg][:Skv], rc.reshape(Skv, D // 2))
        assert np.array_equal(ks[bg][:Skv], rs.reshape(Skv, D // 32))
        assert not kc[bg][Skv:].any() and not ks[bg][Skv:].any()
        rc, rs = oracle.quantize_t(v.reshape(B * Hkv, Skv, D)[bg], rule)
        assert np.array_equal(vc[bg][:, :pad32 // 2], rc)
        assert np.array_equal(vs[bg][:, :pad32 // 32], rs)
        assert not vc[bg][:, pad32 // 2:].any() and not vs[bg][:, pad32 // 32:].any()


def run_case(q, k, v, causal, mode, rows=None, check_ws=True, label=""):
    torch, mx = gpu()
    print(f"[case] {label} mode={mode} causal={causal} q={q.shape} k={k.shape} "
          f"dtype={q.dtype}", flush=True)
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    if rows is None:
        rows = np.arange(B * Hq * Sq, dtype=np.int64)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    ws = mx.alloc_workspace(qt, kt, mode)
    o = mx.attn_fwd(qt, kt, vt, causal=causal, mode=mode, workspace=ws)
    torch.cuda.synchronize()
    if check_ws and mode != "fp16":
        check_workspace(mx, ws, q, k, v, mode, with_q=False)
    bc = mx.kv_tile(D, mode)
    rq, rk, rv = q, k, v
    if mode == "fp16" and q.dtype == np.float32:
        # FP16 mode's operands are 16-bit: fp32 inputs enter as fp16 Q, K and
        # V, so the reference takes the same rounded operands (the remaining
        # difference is P's fp16 rounding and the accumulation order); bf16
        # inputs are used as they are (V's bf16 -> fp16 conversion is exact
        # in fp16's normal range)
        rq, rk, rv = (a.astype(np.float16).astype(np.float32) for a in (q, k, v))
    ref = oracle.attn_rows(rq, rk, rv, causal=causal, mode=MODE_IDS[mode], bc=bc, rows=rows,
                           want_p=(mode != "fp16"))
    got = o.reshape(-1, D)[torch.from_numpy(rows).to(o.device)].double().cpu().numpy()
    err = np.abs(got - ref["o"])
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean())}
    if mode != "fp16":
        o2, pc, ps, ws2 = mx.attn_fwd_dump(qt, kt, vt, rows, causal=causal, mode=mode)
        assert torch.equal(o2, o), "dump variant changed O"
        if check_ws:
            check_workspace(mx, ws2, q, k, v, mode, with_q=True)
        fr, sfr, nflip = flips(np_u8(pc), np_u8(ps), ref["p_codes"], ref["p_scales"], Skv)
        stats.update(flip_frac=fr, scale_flip_frac=sfr, nflip=nflip)
        assert fr <= FLIP_MAX, stats
    print(f"[case] {label} {mode}: {stats}", flush=True)
    assert stats["max_abs"] <= MAX_ABS, stats
    assert stats["mean_abs"] <= MEAN_ABS, stats
    return o, stats


def bf16_qkv(seed, B, Hq, Hkv, Sq, Skv, D, scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, Sq, D)) * scale).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, Skv, D)) * scale).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    return tuple(mxsynth.f32_to_bf16_bits(t) for t in (q, k, v))


# ---------------------------------------------------------------- small ----

@pytest.mark.parametrize("mode", ALL_MODES)
def test_tiny_config(mode):
    q, k, v = mxsynth.tiny_attn(0)
    run_case(q, k, v, False, mode, label="tiny")


@pytest.mark.parametrize("mode", ALL_MODES)
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_gqa(mode, causal):
    q, k, v = bf16_qkv(11, 2, 4, 2, 300, 300, 128, scale=1.3)
    run_case(q, k, v, causal, mode, label="ragged_gqa")


@pytest.mark.parametrize("mode", ALL_MODES)
def test_rect_noncausal(mode):
    q, k, v = bf16_qkv(12, 1, 2, 1, 200, 333, 128)
    run_case(q, k, v, False, mode, label="rect")


@pytest.mark.parametrize("mode", ALL_MODES)
def test_d64_bf16(mode):
    q, k, v = bf16_qkv(13, 1, 3, 3, 130, 130, 64, scale=1.5)
    run_case(q, k, v, True, mode, label="d64")


@pytest.mark.parametrize("mode", ALL_MODES)
def test_fp32_d128(mode):
    """fp32 inputs at D = 128 (the MX kernels quantize fp32 query rows; FP16
    mode converts Q and K to fp16 and runs S^T on the fp16 matrix cores;
    ragged query and key ends)."""
    rng = np.random.default_rng(15)
    q = (rng.standard_normal((1, 2, 190, 128)) * 1.4).astype(np.float32)
    k = (rng.standard_normal((1, 2, 261, 128)) * 1.4).astype(np.float32)
    v = rng.standard_normal((1, 2, 261, 128)).astype(np.float32)
    run_case(q, k, v, False, mode, label="fp32_d128")


@pytest.mark.parametrize("mode", ALL_MODES)
@pytest.mark.parametrize("D", [64, 128])
def test_fp32_causal(mode, D):
    """fp32 inputs, causal, GQA, a ragged length that leaves a partial last
    query tile and a partial last KV tile."""
    rng = np.random.default_rng(16 + D)
    q = (rng.standard_normal((1, 4, 333, D)) * 1.2).astype(np.float32)
    k = (rng.standard_normal((1, 2, 333, D)) * 1.2).astype(np.float32)
    v = rng.standard_normal((1, 2, 333, D)).astype(np.float32)
    run_case(q, k, v, True, mode, label=f"fp32_causal_d{D}")


@pytest.mark.parametrize("shape", [(1, 1), (5, 1), (1, 1000), (33, 33), (129, 129)])
@pytest.mark.parametrize("mode", ["fp16", "uos_pnq", "ocp", "uos_efq"])
def test_edge_lengths(shape, mode):
    Sq, Skv = shape
    q, k, v = bf16_qkv(14, 1, 2, 2, Sq, Skv, 128)
    run_case(q, k, v, False, mode, label=f"edge{shape}")
    if Sq == Skv:
        run_case(q, k, v, True, mode, label=f"edge{shape}-causal")


@pytest.mark.parametrize("mode", ALL_MODES)
def test_dit_like_small(mode):
    """Outlier channels x20 and a smooth per-token bias, at a small size."""
    q, k, v = mxsynth.video_dit(21, H=2, grid=(3, 7, 9))
    run_case(q, k, v, False, mode, label="dit_small")


@pytest.mark.parametrize("mode", MX_MODES)
def test_llm_like_small(mode):
    q, k, v = mxsynth.llm_prefill(22, B=1, Hq=8, Hkv=2, S=257)
    run_case(q, k, v, True, mode, label="llm_small")


def test_v_ones_pnq_gives_one():
    """Under PNQ (and EFQ, which shares its denominator) numerator and
    denominator sum the same P~, so O = 1 up to fp32 accumulation rounding;
    the non-PNQ modes divide sum(P~) by sum(P) and miss 1 by far more."""
    torch, mx = gpu()
    q, k, v = bf16_qkv(15, 1, 2, 2, 190, 190, 128, scale=2.0)
    v[:] = mxsynth.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    dev = {m: (mx.attn_fwd(qt, kt, vt, mode=m) - 1.0).abs().max().item()
           for m in ("uos_pnq", "uos_efq", "uos", "ocp")}
    print("max |O - 1|:", dev)
    assert dev["uos_pnq"] <= 1e-6 and dev["uos_efq"] <= 1e-6
    assert dev["uos"] > 1e-3 and dev["ocp"] > 1e-3


def test_q_zero_gives_mean_v():
    torch, mx = gpu()
    q, k, v = bf16_qkv(16, 1, 2, 2, 64, 300, 128)
    q[:] = 0
    run_case(q, k, v, False, "uos_pnq", label="q0")


@pytest.mark.parametrize("mode", ALL_MODES)
def test_deterministic(mode):
    torch, mx = gpu()
    q, k, v = bf16_qkv(17, 1, 4, 4, 700, 700, 128)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    a = mx.attn_fwd(qt, kt, vt, mode=mode)
    b = mx.attn_fwd(qt, kt, vt, mode=mode)
    assert torch.equal(a, b)


# ----------------------------------------------------------- full sizes ----

@functools.lru_cache(maxsize=1)
def full_inputs(name):
    return mxsynth.make_attn_inputs(name)


@pytest.mark.slow
@pytest.mark.parametrize("mode", MX_MODES)
def test_full_llm_prefill(mode):
    c = mxsynth.CONFIGS["llm_prefill"]
    q, k, v = full_inputs("llm_prefill")
    rows = mxsynth.sample_rows(c["seed"], c["B"], c["Hq"], c["S"], 256)
    run_case(q, k, v, True, mode, rows=rows, check_ws=(mode == "uos_pnq"), label="llm_prefill")


@pytest.mark.slow
@pytest.mark.parametrize("mode", ALL_MODES)
def test_full_dit14(mode):
    c = mxsynth.CONFIGS["dit14"]
    q, k, v = full_inputs("dit14")
    rows = mxsynth.sample_rows(c["seed"], c["B"], c["Hq"], c["S"], 256)
    run_case(q, k, v, False, mode, rows=rows, check_ws=(mode == "uos_pnq"), label="dit14")


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["uos_pnq", "uos_efq", "ocp", "fp16"])
def test_full_dit13(mode):
    c = mxsynth.CONFIGS["dit13"]
    q, k, v = full_inputs("dit13")
    rows = mxsynth.sample_rows(c["seed"], c["B"], c["Hq"], c["S"], 256)
    run_case(q, k, v, False, mode, rows=rows, check_ws=False, label="dit13")
