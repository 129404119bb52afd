"""GPU parity of the per-sequence-length forms (``mxattn_fwd_varlen``,
``mxattn_decode_varlen``) against the binary64 oracle run on each batch
entry's own rows and keys (the oracle needs no notion of a batch of
lengths: entry b is attention on q[b, :, :len_q], k[b, :, :len_k],
v[b, :, :len_k]).

Bars as for mxattn_fwd: O max-abs <= 2e-3 and mean-abs <= 2e-4 per entry;
P~ flip fraction <= 1e-4 (dump of every valid row); the kernel's Q~ of the
valid rows bit-exact.  The padding past each entry's lengths holds NaN, so
any key, value or query row read past a length would poison the result;
rows past an entry's query length (or with no visible key) keep the
sentinel that ``out`` was filled with.  With every length at its maximum
the varlen forms give the same O bits as mxattn_fwd / mxattn_decode.
"""
import numpy as np
import pytest

from common import (FLIP_MAX, MAX_ABS, MEAN_ABS, MODE_IDS, RULE_IDS, RULE_OF_MODE, flips, gpu,
                    mxsynth, np_u8, oracle, to_torch)

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0
NAN_BF16 = np.uint16(0x7FC0)


def padded_inputs(seed, B, Hq, Hkv, Sq, Skv, D, lens_q, lens_k, scale=1.3):
    """bf16 q, k, v with NaN past each entry's lengths."""
    rng = np.random.default_rng(seed)
    q = mxsynth.f32_to_bf16_bits((rng.standard_normal((B, Hq, Sq, D)) * scale).astype(np.float32))
    k = mxsynth.f32_to_bf16_bits((rng.standard_normal((B, Hkv, Skv, D)) * scale).astype(np.float32))
    v = mxsynth.f32_to_bf16_bits(rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32))
    for b in range(B):
        q[b, :, lens_q[b]:] = NAN_BF16
        k[b, :, lens_k[b]:] = NAN_BF16
        v[b, :, lens_k[b]:] = NAN_BF16
    return q, k, v


def compare_entry(o, pc, ps, b, rows_b, q, k, v, lq, lk, causal, mode, split, label):
    """Entry b against the oracle on its own rows and keys; returns stats."""
    D = q.shape[3]
    sel = np.arange(q.shape[1] * lq, dtype=np.int64)
    ref = oracle.attn_rows(q[b:b + 1, :, :lq], k[b:b + 1, :, :lk], v[b:b + 1, :, :lk],
                           causal=causal, mode=MODE_IDS[mode], bc=128, rows=sel, want_p=True,
                           split=split)
    got = o[b][:, :lq].reshape(-1, D)
    err = np.abs(got - ref["o"])
    fr, sfr, nflip = flips(pc[rows_b], ps[rows_b], ref["p_codes"], ref["p_scales"], lk)
    st = {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "flip_frac": fr,
          "nflip": nflip}
    print(f"[case] {label} b={b} lq={lq} lk={lk}: {st}", flush=True)
    assert fr <= FLIP_MAX, st
    assert st["max_abs"] <= MAX_ABS and st["mean_abs"] <= MEAN_ABS, st


def check_q_tilde(ws, mx, q, lens_q, B, Hq, Hkv, Sq, Skv, D, mode):
    off, _ = mx.workspace_layout(B, Hq, Hkv, Sq, Skv, D, "bf16", mode)
    w = np_u8(ws)
    rule = RULE_IDS[RULE_OF_MODE[mode]]
    codes = w[off[0]:off[0] + B * Hq * Sq * D // 2].reshape(B, Hq, Sq, D // 2)
    scales = w[off[1]:off[1] + B * Hq * Sq * D // 32].reshape(B, Hq, Sq, D // 32)
    for b in range(B):
        rc, rs = oracle.quantize(q[b, :, :lens_q[b]], rule)
        assert np.array_equal(codes[b, :, :lens_q[b]].reshape(-1), rc)
        assert np.array_equal(scales[b, :, :lens_q[b]].reshape(-1), rs)


def flat_rows(Hq, Sq, lens_q, B):
    """Flattened (b*Hq + h)*Sq + i of every valid row, and per entry the
    positions of its rows inside that list (h-major, the oracle's order)."""
    rows, pos, n = [], [], 0
    for b in range(B):
        r = np.array([(b * Hq + h) * Sq + i for h in range(Hq) for i in range(lens_q[b])],
                     dtype=np.int64)
        pos.append(np.arange(n, n + r.size))
        n += r.size
        rows.append(r)
    return np.concatenate(rows), pos


PREFILL = [
    # (B, Hq, Hkv, Sq, Skv, D, lens_q, lens_k, causal)
    (3, 4, 2, 300, 333, 128, [300, 1, 129], [333, 77, 129], True),
    (3, 4, 2, 300, 333, 128, [257, 40, 300], [1, 333, 200], False),
    (2, 2, 2, 200, 200, 64, [200, 130], [200, 170], True),
    # empty entries: no query rows; no keys; a causal entry with more rows than keys
    (4, 4, 2, 200, 260, 128, [0, 150, 200, 90], [100, 0, 260, 60], True),
]


@pytest.mark.parametrize("mode", ["ocp", "uos", "uos_pnq", "uos_efq"])
@pytest.mark.parametrize("case", PREFILL)
def test_fwd_varlen(case, mode):
    torch, mx = gpu()
    B, Hq, Hkv, Sq, Skv, D, lq, lk, causal = case
    print(f"[case] fwd_varlen {case} {mode}", flush=True)
    q, k, v = padded_inputs(70 + Sq + D, B, Hq, Hkv, Sq, Skv, D, lq, lk)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    rows, pos = flat_rows(Hq, Sq, lq, B)
    out = torch.full((B, Hq, Sq, D), SENTINEL, dtype=torch.float32, device="cuda")
    o, pc, ps, ws = mx.attn_fwd_varlen(qt, kt, vt, lq, lk, causal=causal, mode=mode, out=out,
                                       rows=rows)
    o = o.double().cpu().numpy()
    pc, ps = np_u8(pc), np_u8(ps)
    for b in range(B):
        if lk[b] == 0 or (causal and lq[b] > lk[b]):
            # no row of this entry sees a key: nothing is written
            assert np.all(o[b] == SENTINEL), "an entry without visible keys was written"
            continue
        assert np.all(o[b][:, lq[b]:] == SENTINEL), "row past the query length written"
        if lq[b] == 0:
            continue
        compare_entry(o, pc, ps, b, pos[b], q, k, v, lq[b], lk[b], causal, mode, 0,
                      f"fwd_varlen {mode}")
    # the kernel quantizes the rows of the entries that write rows
    eff = [lq[b] if lk[b] > 0 and not (causal and lq[b] > lk[b]) else 0 for b in range(B)]
    check_q_tilde(ws, mx, q, eff, B, Hq, Hkv, Sq, Skv, D, mode)


@pytest.mark.parametrize("mode", ["uos_pnq", "uos_efq"])
def test_varlen_fp32_inputs(mode):
    """fp32 inputs (NaN past each length): the kernels quantize fp32 query
    rows in their prologue and the image quantizer fp32 keys and values
    under the lengths; prefill (non-causal) and decode (causal)."""
    torch, mx = gpu()
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 190, 261, 128
    lq, lk = [190, 77], [261, 100]
    rng = np.random.default_rng(33)
    q = (rng.standard_normal((B, Hq, Sq, D)) * 1.4).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, Skv, D)) * 1.4).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    for b in range(B):
        q[b, :, lq[b]:] = np.nan
        k[b, :, lk[b]:] = np.nan
        v[b, :, lk[b]:] = np.nan
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    rows, pos = flat_rows(Hq, Sq, lq, B)
    out = torch.full((B, Hq, Sq, D), SENTINEL, dtype=torch.float32, device="cuda")
    o, pc, ps, ws = mx.attn_fwd_varlen(qt, kt, vt, lq, lk, causal=False, mode=mode, out=out,
                                       rows=rows)
    o = o.double().cpu().numpy()
    pc, ps = np_u8(pc), np_u8(ps)
    for b in range(B):
        assert np.all(o[b][:, lq[b]:] == SENTINEL), "row past the query length written"
        compare_entry(o, pc, ps, b, pos[b], q, k, v, lq[b], lk[b], False, mode, 0,
                      f"varlen_fp32 {mode}")
    # decode: two query rows per entry against the same cache, causal
    qd = np.ascontiguousarray(q[:, :, :2])
    out_d = mx.attn_decode_varlen(to_torch(qd), kt, vt, lk, causal=True, mode=mode)
    od = out_d.double().cpu().numpy()
    split = mx.decode_split(B, Hkv, Skv)
    for b in range(B):
        ref = oracle.attn_rows(qd[b:b + 1], k[b:b + 1, :, :lk[b]], v[b:b + 1, :, :lk[b]],
                               causal=True, mode=MODE_IDS[mode], bc=128,
                               rows=np.arange(Hq * 2, dtype=np.int64), split=split)
        err = np.abs(od[b].reshape(-1, D) - ref["o"])
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (b, err.max())


def test_fwd_varlen_full_lengths_match_fwd():
    torch, mx = gpu()
    B, Hq, Hkv, S, D = 2, 4, 2, 300, 128
    q, k, v = padded_inputs(80, B, Hq, Hkv, S, S, D, [S] * B, [S] * B)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    for causal in (False, True):
        a = mx.attn_fwd(qt, kt, vt, causal=causal, mode="uos_pnq")
        b = mx.attn_fwd_varlen(qt, kt, vt, [S] * B, [S] * B, causal=causal, mode="uos_pnq")
        assert torch.equal(a, b)


DECODE = [
    # (B, Hq, Hkv, Sq, Skv, D, lens_k, causal)
    (4, 8, 2, 2, 5000, 128, [5000, 1, 2000, 129], True),
    (3, 4, 4, 1, 3000, 64, [3000, 64, 1500], False),
    (2, 16, 2, 2, 2500, 128, [2400, 700], True),
    (3, 8, 2, 1, 3000, 128, [0, 3000, 700], True),  # an empty cache: its rows stay unwritten
]


@pytest.mark.parametrize("mode", ["ocp", "uos_pnq", "uos_efq"])
@pytest.mark.parametrize("case", DECODE)
def test_decode_varlen(case, mode):
    torch, mx = gpu()
    B, Hq, Hkv, Sq, Skv, D, lk, causal = case
    print(f"[case] decode_varlen {case} {mode}", flush=True)
    q, k, v = padded_inputs(90 + Skv + D, B, Hq, Hkv, Sq, Skv, D, [Sq] * B, lk)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    split = mx.decode_split(B, Hkv, Skv)
    # rows that see a key: causal row i sees keys j <= i + lk - Sq
    first = [min(max(Sq - l, 0), Sq) if causal else 0 for l in lk]
    first = [Sq if l == 0 else f for f, l in zip(first, lk)]
    rows, pos = flat_rows(Hq, Sq, [Sq] * B, B)
    out = torch.full((B, Hq, Sq, D), SENTINEL, dtype=torch.float32, device="cuda")
    o, pc, ps, _ = mx.attn_decode_varlen(qt, kt, vt, lk, causal=causal, mode=mode, out=out,
                                         rows=rows)
    # the prepared pair (KV cache quantized once) gives the same bits
    ws2 = mx.attn_prepare_varlen(qt, kt, vt, lk, mode=mode)
    out2 = torch.full((B, Hq, Sq, D), SENTINEL, dtype=torch.float32, device="cuda")
    o2 = mx.attn_decode_varlen_prepared(qt, kt, ws2, lk, causal=causal, mode=mode, out=out2)
    assert torch.equal(o2, o), "prepared varlen decode differs"
    o = o.double().cpu().numpy()
    pc, ps = np_u8(pc), np_u8(ps)
    for b in range(B):
        f = first[b]
        assert np.all(o[b][:, :f] == SENTINEL), "a row with no visible key was written"
        if f == Sq:
            continue
        # the rows that see keys, as an oracle problem of Sq - f rows
        keep = np.array([h * Sq + i for h in range(Hq) for i in range(f, Sq)], dtype=np.int64)
        ref = oracle.attn_rows(q[b:b + 1, :, f:], k[b:b + 1, :, :lk[b]], v[b:b + 1, :, :lk[b]],
                               causal=causal, mode=MODE_IDS[mode], bc=128,
                               rows=np.arange(keep.size, dtype=np.int64), want_p=True, split=split)
        got = o[b][:, f:].reshape(-1, D)
        err = np.abs(got - ref["o"])
        rb = pos[b][keep]
        fr, _, nflip = flips(pc[rb], ps[rb], ref["p_codes"], ref["p_scales"], lk[b])
        st = {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "flip_frac": fr,
              "nflip": nflip}
        print(f"[case] decode_varlen {mode} b={b} lk={lk[b]}: {st}", flush=True)
        assert fr <= FLIP_MAX, st
        assert st["max_abs"] <= MAX_ABS and st["mean_abs"] <= MEAN_ABS, st


@pytest.mark.parametrize("B", [130, 300])
def test_decode_varlen_many_entries(B):
    """Batches past one 64-entry step of the busy-split scan (130 entries:
    three steps) and past the scan's limit of 256 entries (300: every split
    of the padded extent numbered); lengths uniform on [0, Skv] with a fifth
    of the entries empty, causal, two splits per full entry."""
    torch, mx = gpu()
    Hq, Hkv, Sq, Skv, D = 2, 1, 1, 700, 64
    rng = np.random.default_rng(500 + B)
    lk = [int(x) for x in rng.integers(0, Skv + 1, B)]
    for b in rng.choice(B, B // 5, replace=False):
        lk[b] = 0
    print(f"[case] decode_varlen_many_entries B={B}", flush=True)
    q, k, v = padded_inputs(600 + B, B, Hq, Hkv, Sq, Skv, D, [Sq] * B, lk)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    split = mx.decode_split(B, Hkv, Skv)
    assert split < Skv  # entries hold up to two splits
    out = torch.full((B, Hq, Sq, D), SENTINEL, dtype=torch.float32, device="cuda")
    o = mx.attn_decode_varlen(qt, kt, vt, lk, causal=True, mode="uos_pnq", out=out)
    o = o.double().cpu().numpy()
    for b in range(B):
        if lk[b] == 0:
            assert np.all(o[b] == SENTINEL), "an entry with no key was written"
            continue
        ref = oracle.attn_rows(q[b:b + 1], k[b:b + 1, :, :lk[b]], v[b:b + 1, :, :lk[b]],
                               causal=True, mode=oracle.MODE_UOS_PNQ, bc=128,
                               rows=np.arange(Hq * Sq, dtype=np.int64), split=split)
        err = np.abs(o[b].reshape(-1, D) - ref["o"])
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (b, lk[b], err.max())


def test_decode_varlen_full_lengths_match_decode():
    torch, mx = gpu()
    B, Hq, Hkv, Sq, Skv, D = 3, 8, 2, 1, 4100, 128
    q, k, v = padded_inputs(95, B, Hq, Hkv, Sq, Skv, D, [Sq] * B, [Skv] * B)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    a = mx.attn_decode(qt, kt, vt, causal=True, mode="uos_pnq")
    b = mx.attn_decode_varlen(qt, kt, vt, [Skv] * B, causal=True, mode="uos_pnq")
    assert torch.equal(a, b)


# ----------------------------------------------------------- full sizes ----

@pytest.mark.slow
def test_full_llm_prefill_varlen():
    """The bench's llm_prefill_varlen call (the llm_prefill tensors, the
    seeded per-entry lengths, causal, UOS+PNQ); 64 seeded rows per (entry,
    head) against the oracle on the entry's own rows and keys.  The padding
    holds the generator's data, which must not leak in."""
    torch, mx = gpu()
    vc = mxsynth.VARLEN_CONFIGS["llm_prefill_varlen"]
    c = mxsynth.CONFIGS[vc["base"]]
    B, Hq, S, D = c["B"], c["Hq"], c["S"], c["D"]
    lens = [int(x) for x in mxsynth.seq_lengths(vc["lens_seed"], B, vc["lo"], vc["hi"])]
    print(f"[case] llm_prefill_varlen lengths {lens}", flush=True)
    q, k, v = mxsynth.make_attn_inputs(vc["base"])
    out = mx.attn_fwd_varlen(to_torch(q), to_torch(k), to_torch(v), lens, lens, causal=True,
                             mode="uos_pnq")
    o = out.cpu().numpy()
    rng = np.random.default_rng(vc["lens_seed"] + 100)
    for b in range(B):
        n = lens[b]
        sel = np.concatenate([h * n + np.sort(rng.choice(n, 64, replace=False))
                              for h in range(Hq)]).astype(np.int64)
        ref = oracle.attn_rows(q[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                               causal=True, mode=oracle.MODE_UOS_PNQ, bc=128, rows=sel)
        got = o[b][:, :n].reshape(-1, D)[sel].astype(np.float64)
        err = np.abs(got - ref["o"])
        print(f"[case] llm_prefill_varlen b={b} len={n}: max {err.max():.3e} mean {err.mean():.3e}",
              flush=True)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
        assert np.all(o[b][:, n:] == 0.0), "row past the length written"


@pytest.mark.slow
def test_full_llm_decode_varlen():
    """The bench's llm_decode_varlen call (the llm_decode cache with the
    seeded per-entry lengths, UOS+PNQ, through the prepared pair); every
    query row against the oracle with the library's split size."""
    torch, mx = gpu()
    vc = mxsynth.VARLEN_CONFIGS["llm_decode_varlen"]
    c = mxsynth.DECODE_CONFIGS[vc["base"]]
    B, Hq, Hkv, Sq, Skv, D = c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Skv"], c["D"]
    lens = [int(x) for x in mxsynth.seq_lengths(vc["lens_seed"], B, vc["lo"], vc["hi"])]
    print(f"[case] llm_decode_varlen lengths {lens}", flush=True)
    q, k, v = mxsynth.llm_decode(c["seed"], B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D)
    qt, kt, vt = to_torch(q), to_torch(k), to_torch(v)
    ws = mx.attn_prepare_varlen(qt, kt, vt, lens, mode="uos_pnq")
    o = mx.attn_decode_varlen_prepared(qt, kt, ws, lens, causal=True, mode="uos_pnq").cpu().numpy()
    split = mx.decode_split(B, Hkv, Skv)
    for b in range(B):
        n = lens[b]
        ref = oracle.attn_rows(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], causal=True,
                               mode=oracle.MODE_UOS_PNQ, bc=128,
                               rows=np.arange(Hq * Sq, dtype=np.int64), split=split)
        err = np.abs(o[b].reshape(-1, D).astype(np.float64) - ref["o"])
        print(f"[case] llm_decode_varlen b={b} len={n}: max {err.max():.3e} mean {err.mean():.3e}",
              flush=True)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
