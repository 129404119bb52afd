"""GPU parity of short-query attention over key splits (``mxattn_decode``)
against the binary64 oracle run with the same split schedule.

Bars as for mxattn_fwd: O max-abs <= 2e-3 and mean-abs <= 2e-4; the P~
codes and E8M0 bytes read back through the dump entry point differ from the
oracle's in at most 1e-4 of the elements; the dump variant and the prepared
variant give the same O bits as the plain call; the Q~ the split kernel forms
(stored by the dump variant) is bit-exact against the oracle's quantizer.
"""
import functools

import numpy as np
import pytest

from common import (FLIP_MAX, MAX_ABS, MEAN_ABS, MODE_IDS, RULE_IDS, RULE_OF_MODE, flips, gpu,
                    mxsynth, np_u8, to_torch)
import oracle

pytestmark = pytest.mark.gpu

MX_MODES = ["ocp", "uos", "uos_pnq", "uos_efq"]


def run_decode(q, k, v, causal, mode, rows=None, label=""):
    torch, mx = gpu()
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    split = mx.decode_split(B, Hkv, Skv)
    print(f"[case] decode {label} mode={mode} causal={causal} q={q.shape} k={k.shape} "
          f"split={split}", flush=True)
    if rows is None:
        rows = np.arange(B * Hq * Sq, dtype=np.int64)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    o = mx.attn_decode(qt, kt, vt, causal=causal, mode=mode)
    o2, pc, ps, ws = mx.attn_decode_dump(qt, kt, vt, rows, causal=causal, mode=mode)
    assert torch.equal(o, o2), "dump variant changed O"
    # the split kernel's own Q~ (stored by the dump variant) is the quantizer's
    off, _ = mx.workspace_layout(B, Hq, Hkv, Sq, Skv, D,
                                 "bf16" if q.dtype == np.uint16 else "f32", mode)
    w = np_u8(ws)
    rc, rs = oracle.quantize(q, RULE_IDS[RULE_OF_MODE[mode]])
    assert np.array_equal(w[off[0]:off[0] + rc.size], rc)
    assert np.array_equal(w[off[1]:off[1] + rs.size], rs)
    mx.attn_prepare(qt, kt, vt, mode=mode, workspace=ws)
    o3 = mx.attn_decode_prepared(qt, kt, ws, causal=causal, mode=mode)
    assert torch.equal(o, o3), "prepared variant changed O"
    ref = oracle.attn_rows(q, k, v, causal=causal, mode=MODE_IDS[mode], bc=128, rows=rows,
                           want_p=True, split=split)
    got = o.reshape(-1, D)[torch.from_numpy(rows).to(o.device)].double().cpu().numpy()
    err = np.abs(got - ref["o"])
    fr, sfr, nflip = flips(np_u8(pc), np_u8(ps), ref["p_codes"], ref["p_scales"], Skv)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "flip_frac": fr,
             "scale_flip_frac": sfr, "nflip": nflip}
    print(f"[case] decode {label} {mode}: {stats}", flush=True)
    assert fr <= FLIP_MAX, stats
    assert stats["max_abs"] <= MAX_ABS, stats
    assert stats["mean_abs"] <= MEAN_ABS, stats
    return o


SMALL = [
    # (B, Hq, Hkv, Sq, Skv, D, causal)
    (1, 8, 2, 1, 1000, 128, True),      # 4 heads x 1 query per group
    (2, 4, 4, 4, 700, 64, False),       # MHA, 4 queries
    (1, 16, 2, 2, 2049, 128, True),     # 16 query columns, ragged keys
    (1, 8, 8, 16, 4097, 128, True),     # last split (key 4096) empty for rows 0..14
    (3, 6, 2, 5, 1300, 64, True),       # 15 columns
    (1, 32, 4, 4, 1500, 128, True),     # 32 query columns (the whole tile)
    (2, 8, 1, 3, 900, 64, False),       # 24 columns, one KV head
]


@pytest.mark.parametrize("mode", MX_MODES)
@pytest.mark.parametrize("shape", SMALL)
def test_small_decode(shape, mode):
    B, Hq, Hkv, Sq, Skv, D, causal = shape
    q, k, v = mxsynth.llm_decode(40 + Skv, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D)
    run_decode(q, k, v, causal, mode, label=f"{shape}")


@pytest.mark.parametrize("mode", ["ocp", "uos_pnq"])
def test_decode_fp32_inputs(mode):
    """fp32 q, k, v: the split kernel quantizes fp32 query rows (the other
    cases are bf16); values off the bf16 grid, scaled so some blocks need
    the UOS step-up."""
    rng = np.random.default_rng(53)
    B, Hq, Hkv, Sq, Skv, D = 2, 8, 2, 3, 1500, 128
    q = (rng.standard_normal((B, Hq, Sq, D)) * 1.7).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, Skv, D)) * 1.3).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    run_decode(q, k, v, True, mode, label="fp32")


def test_decode_single_key_and_v_ones():
    torch, mx = gpu()
    # one key: O is that key's quantized value row
    q, k, v = mxsynth.llm_decode(50, B=1, Hq=4, Hkv=1, Sq=1, Skv=1, D=128)
    run_decode(q, k, v, True, "uos_pnq", label="one key")
    # V = 1 under PNQ (and EFQ): O = 1 up to fp32 rounding, through the merge
    q, k, v = mxsynth.llm_decode(51, B=1, Hq=8, Hkv=2, Sq=2, Skv=3000, D=128)
    v[:] = mxsynth.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    for mode in ("uos_pnq", "uos_efq"):
        o = mx.attn_decode(to_torch(q), to_torch(k), to_torch(v), causal=True, mode=mode)
        assert (o - 1.0).abs().max().item() <= 1e-5


def test_decode_deterministic():
    torch, mx = gpu()
    q, k, v = mxsynth.llm_decode(52, B=2, Hq=8, Hkv=2, Sq=1, Skv=5000, D=128)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    a = mx.attn_decode(qt, kt, vt, causal=True, mode="uos_pnq")
    b = mx.attn_decode(qt, kt, vt, causal=True, mode="uos_pnq")
    assert torch.equal(a, b)


def test_decode_arrival_counters():
    """The split kernel counts each group's finished splits in the workspace
    and the last one merges.  The counters are cleared with the KV images
    (so a workspace filled with junk beforehand works) and left at zero by
    every call, so consecutive prepared calls on one workspace, including
    per-entry lengths with an empty entry (no split of it, nothing counted),
    equal the same calls on fresh workspaces bit for bit; the largest split
    count (1024 splits, 64 merge chunks) is covered too."""
    torch, mx = gpu()
    q, k, v = mxsynth.llm_decode(53, B=3, Hq=8, Hkv=2, Sq=2, Skv=5000, D=128)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    print("[case] decode counters: junk workspace, consecutive prepared calls", flush=True)
    ws = mx.alloc_decode_workspace(qt, kt, "uos_pnq")
    ws.fill_(0xFF)
    ref = mx.attn_decode(qt, kt, vt, causal=True, mode="uos_pnq")
    assert torch.equal(mx.attn_decode(qt, kt, vt, causal=True, mode="uos_pnq", workspace=ws), ref)
    for i in range(3):
        qi = to_torch(mxsynth.llm_decode(54 + i, B=3, Hq=8, Hkv=2, Sq=2, Skv=5000, D=128)[0])
        want = mx.attn_decode(qi, kt, vt, causal=i % 2 == 0, mode="uos_pnq")
        got = mx.attn_decode_prepared(qi, kt, ws, causal=i % 2 == 0, mode="uos_pnq")
        assert torch.equal(got, want), f"prepared call {i}"
    lens = [0, 3001, 5000]
    wsv = mx.alloc_decode_workspace(qt, kt, "uos_efq")
    wsv.fill_(0xFF)
    mx.attn_prepare_varlen(qt, kt, vt, lens, mode="uos_efq", workspace=wsv)
    want = mx.attn_decode_varlen(qt, kt, vt, lens, causal=True, mode="uos_efq")
    for i in range(3):
        got = mx.attn_decode_varlen_prepared(qt, kt, wsv, lens, causal=True, mode="uos_efq")
        assert torch.equal(got, want), f"prepared per-entry-length call {i}"
    assert not got[0].any(), "the entry with no key wrote rows"
    # one group over 1024 splits of 8 tiles
    q1, k1, v1 = mxsynth.llm_decode(57, B=1, Hq=4, Hkv=1, Sq=1, Skv=1 << 20, D=64)
    q1t, k1t, v1t = to_torch(q1), to_torch(k1), to_torch(v1)
    assert mx.decode_split(1, 1, 1 << 20) == 1024
    print("[case] decode counters: 1024 splits", flush=True)
    a = mx.attn_decode(q1t, k1t, v1t, causal=False, mode="uos_pnq")
    ws1 = mx.attn_prepare(q1t, k1t, v1t, mode="uos_pnq",
                          workspace=mx.alloc_decode_workspace(q1t, k1t, "uos_pnq"))
    for i in range(2):
        assert torch.equal(mx.attn_decode_prepared(q1t, k1t, ws1, mode="uos_pnq"), a)
    rows = np.arange(4, dtype=np.int64)
    ref1 = oracle.attn_rows(q1, k1, v1, causal=False, mode=MODE_IDS["uos_pnq"], bc=128,
                            rows=rows, split=mx.decode_split(1, 1, 1 << 20))
    err = np.abs(a.reshape(-1, 64).double().cpu().numpy() - ref1["o"])
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


@functools.lru_cache(maxsize=1)
def full_inputs(name):
    c = mxsynth.DECODE_CONFIGS[name]
    return mxsynth.llm_decode(c["seed"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], Sq=c["Sq"],
                              Skv=c["Skv"], D=c["D"])


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["uos_pnq", "uos_efq", "ocp"])
def test_full_llm_decode(mode):
    c = mxsynth.DECODE_CONFIGS["llm_decode"]
    q, k, v = full_inputs("llm_decode")
    # every query of batch items 0 and B-1
    per_b = c["Hq"] * c["Sq"]
    rows = np.r_[np.arange(per_b), np.arange((c["B"] - 1) * per_b, c["B"] * per_b)].astype(np.int64)
    run_decode(q, k, v, c["causal"], mode, rows=rows, label="llm_decode")
