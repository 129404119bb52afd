"""The C ABI's stream argument: every call is enqueued on the stream it is
given (a side stream, a graph-capturing stream), and the library neither
allocates, synchronizes nor issues memsets, so the attention, short-query
attention, W4A4 product, quantizer and per-sequence-length calls can be
captured into one HIP graph and replayed.

Checked: results on a side stream (inputs produced on that same stream just
before the call) equal the default-stream results bit for bit; a captured
graph replayed several times, with eager work on the device between the
replays, reproduces the eager results every time.
"""
import numpy as np
import pytest

from common import gpu, mxsynth, to_torch

pytestmark = pytest.mark.gpu


def qkv(seed, B, Hq, Hkv, Sq, Skv, D):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, Sq, D)) * 1.3).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, Skv, D)) * 1.3).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Skv, D)).astype(np.float32)
    return tuple(to_torch(mxsynth.f32_to_bf16_bits(t)) for t in (q, k, v))


def test_side_stream():
    torch, mx = gpu()
    q, k, v = qkv(60, 1, 4, 2, 300, 300, 128)
    ref = mx.attn_fwd(q, k, v, causal=True, mode="uos_pnq")
    qd, kd, vd = qkv(61, 2, 8, 2, 1, 3000, 128)
    ref_d = mx.attn_decode(qd, kd, vd, causal=True, mode="uos_efq")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # inputs written on s right before the calls that read them
        q2 = q * 1
        out = mx.attn_fwd(q2, k, v, causal=True, mode="uos_pnq", stream=s)
        qd2 = qd * 1
        out_d = mx.attn_decode(qd2, kd, vd, causal=True, mode="uos_efq", stream=s)
    s.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(out_d, ref_d)


def test_stream_argument_not_current():
    """stream=s while another stream is current: the temporaries the binding
    makes (workspace, length arrays, dump buffers, zero-filled outputs) live
    on s, so allocations and fills on the current stream right after the
    call cannot take them over while the kernels still run."""
    torch, mx = gpu()
    q, k, v = qkv(64, 1, 4, 2, 700, 700, 128)
    qd, kd, vd = qkv(65, 2, 8, 2, 1, 6000, 128)
    lq = [640, 600]
    lk = [700, 650]
    q2, k2, v2 = (torch.cat([t, t]) for t in (q, k, v))
    rows = [5, 699, 2 * 700 + 3]
    ref = mx.attn_fwd(q, k, v, causal=True, mode="uos_pnq")
    ref_v = mx.attn_fwd_varlen(q2, k2, v2, lq, lk, causal=True, mode="uos_pnq")
    ref_dump = mx.attn_fwd_dump(q, k, v, rows, causal=False, mode="uos")
    ref_d = mx.attn_decode(qd, kd, vd, causal=True, mode="uos_efq")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    junk = []

    def churn():
        # current-stream allocations and writes while s may still be busy
        for _ in range(4):
            junk.append(torch.full((1 << 24,), 7, dtype=torch.uint8, device="cuda"))

    out = mx.attn_fwd(q, k, v, causal=True, mode="uos_pnq", stream=s)
    churn()
    out_v = mx.attn_fwd_varlen(q2, k2, v2, lq, lk, causal=True, mode="uos_pnq", stream=s)
    churn()
    out_dump = mx.attn_fwd_dump(q, k, v, rows, causal=False, mode="uos", stream=s)
    churn()
    out_d = mx.attn_decode(qd, kd, vd, causal=True, mode="uos_efq", stream=s)
    churn()
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(out_v, ref_v)
    for got, want in zip(out_dump[:3], ref_dump[:3]):
        assert torch.equal(got, want)
    assert torch.equal(out_d, ref_d)


def test_graph_capture_and_replay():
    torch, mx = gpu()
    q, k, v = qkv(62, 1, 4, 2, 260, 260, 128)
    qd, kd, vd = qkv(63, 2, 8, 2, 2, 2500, 64)
    M, N, K = 600, 520, 512
    x, w = mxsynth.w4a4_operands(64, M, N, K)
    xt, wt = to_torch(x), to_torch(w)
    wc, ws = mx.quantize(wt, "uos")

    ws_a = mx.alloc_workspace(q, k, "uos_pnq")
    ws_d = mx.alloc_decode_workspace(qd, kd, "uos_pnq")
    ws_g = mx.gemm_workspace(M, N, K)
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    od = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    # per-sequence lengths (device arrays read by the kernels at run time)
    lq = torch.tensor([253], dtype=torch.int32, device="cuda")
    lk = torch.tensor([260], dtype=torch.int32, device="cuda")
    lk_d = torch.tensor([2500, 1333], dtype=torch.int32, device="cuda")
    ws_v = mx.alloc_workspace(q, k, "uos_pnq")
    ws_dv = mx.alloc_decode_workspace(qd, kd, "uos_efq")
    # KV caches quantized once, outside the graph: the captured short-query
    # calls then rely on their arrival counters returning to 0 after each call
    ws_dp = mx.attn_prepare(qd, kd, vd, mode="uos_pnq",
                            workspace=mx.alloc_decode_workspace(qd, kd, "uos_pnq"))
    ws_dvp = mx.attn_prepare_varlen(qd, kd, vd, lk_d, mode="uos_pnq")
    odp = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    odvp = torch.zeros(qd.shape, dtype=torch.float32, device="cuda")
    ov = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    odv = torch.zeros(qd.shape, dtype=torch.float32, device="cuda")
    xc = torch.empty(M * K // 2, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M * K // 32, dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def work(stream=None):
        mx.attn_fwd(q, k, v, causal=True, mode="uos_pnq", out=o, workspace=ws_a, stream=stream)
        mx.attn_decode(qd, kd, vd, causal=True, mode="uos_pnq", out=od, workspace=ws_d,
                       stream=stream)
        mx.quantize(xt, "uos", xc, xs, stream=stream)
        mx.gemm(xc, xs, wc, ws, M, N, K, out=y, workspace=ws_g, stream=stream)
        mx.attn_fwd_varlen(q, k, v, lq, lk, causal=True, mode="uos_pnq", out=ov,
                           workspace=ws_v, stream=stream)
        mx.attn_decode_varlen(qd, kd, vd, lk_d, causal=True, mode="uos_efq", out=odv,
                              workspace=ws_dv, stream=stream)
        mx.attn_decode_prepared(qd, kd, ws_dp, causal=True, mode="uos_pnq", out=odp,
                                stream=stream)
        mx.attn_decode_varlen_prepared(qd, kd, ws_dvp, lk_d, causal=True, mode="uos_pnq",
                                       out=odvp, stream=stream)

    outs = (o, od, xc, xs, y, ov, odv, odp, odvp)
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work(stream=s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        work(stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_()  # eager device work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"replay {rep}, output {i}"
