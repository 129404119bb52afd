#!/usr/bin/env python3
"""Benchmark of MXFP4 UOS+PNQ attention on one MI355X.

A step is one mxattn_fwd call in UOS+PNQ mode on the long video-DiT 13B
self-attention shape (B=1, H=24, S=118800, D=128, bf16 inputs, non-causal),
the largest configuration that runs on one GPU: quantize K (blocks along D)
and V (blocks along keys), then the fused FP4 attention kernel, which
quantizes Q (blocks along D) as it loads it.  Inputs are seeded synthetic
tensors (mxsynth) already resident in HBM.  Prints ONE JSON line on stdout;
progress goes to stderr.

value      = attention TFLOP/s of the whole step, 4*B*H*Sq*Skv*D / time
             (halved when causal);
roofline   = the fused attention kernel alone, timed with stream events,
             against the 10.1 PFLOP/s dense FP4 MFMA peak;
alongside  = the FP16 (unquantized), OCP and UOS+EFQ (exp-free P~) modes on
             the same inputs;
attention  = the video-DiT 14B shape (B=1, H=40, S=32760) in every mode and
             the causal LLM prefill (B=4, 32 query / 8 KV heads, S=8192) in
             the OCP, UOS, UOS+PNQ and UOS+EFQ modes, whole step and kernel
             alone;
quantizer  = the standalone quantize / dequantize of the 8192 x 28672 bf16
             roundtrip tensor, GB/s against 8 TB/s HBM;
decode     = short-query attention over key splits (mxattn_decode_prepared,
             KV cache already quantized) on one LLM decode step (B=8, 32 query
             / 8 KV heads, 32768 cached keys), GB/s of the quantized KV cache
             read against 8 TB/s; decode.varlen the same cache with per-entry
             lengths (mxattn_decode_varlen_prepared);
prefill_varlen = the LLM prefill batch (B=4, causal) with per-entry prompt
             lengths, one mxattn_fwd_varlen call per step, TFLOP/s of each
             entry's own causal pairs against 10.1 PFLOP/s;
gemm       = the W4A4 product (mxgemm) on the DiT feed-forward up-projection
             (32760 tokens x 5120 -> 13824, UOS operands, bf16 output), alone
             and with the activation quantization, against 10.1 PFLOP/s;
cpu_baseline = the binary64 oracle on a bounded row sample of the headline
             workload, host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 UOS+PNQ attention TFLOPS and % FP4 MFMA peak on 1 MI355X"
FP4_PEAK_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
ATTN_SOURCES = [os.path.join(ROOT, "mxfp4_block_quantized_amd", "csrc", f)
                for f in ("attn_mx.hip", "internal.h", "mx_block.h")]
GEMM_SOURCES = [os.path.join(ROOT, "mxfp4_block_quantized_amd", "csrc", f)
                for f in ("gemm_mx.hip", "internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(sources=ATTN_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def warm(torch, fn, min_ms=200.0, max_calls=5000):
    """Untimed calls of fn until min_ms of wall time has passed (at least
    3): brings the GPU clock back up after host-side input generation."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or ((time.perf_counter() - t0) * 1e3 < min_ms and n < max_calls):
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def attn_flops(c) -> float:
    f = 4.0 * c["B"] * c["Hq"] * c["S"] * c["S"] * c["D"]
    return f / 2 if c["causal"] else f


def time_attention(torch, mx, qt, kt, vt, c, mode, steps, warmup, min_warm_ms=0.0):
    """Returns (ms per whole step, ms of prepare, ms of the attention kernel).
    ``warmup`` untimed steps first (and more, up to ``min_warm_ms`` of wall
    time, for the sections that follow host-side input generation)."""
    causal = c["causal"]
    ws = mx.alloc_workspace(qt, kt, mode)
    out = torch.empty(qt.shape, dtype=torch.float32, device=qt.device)
    for _ in range(warmup):
        mx.attn_fwd(qt, kt, vt, causal=causal, mode=mode, out=out, workspace=ws)
    if min_warm_ms > 0:
        warm(torch, lambda: mx.attn_fwd(qt, kt, vt, causal=causal, mode=mode, out=out,
                                        workspace=ws), min_ms=min_warm_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        mx.attn_prepare(qt, kt, vt, mode=mode, workspace=ws)
        e[1].record()
        mx.attn_fwd_prepared(qt, kt, ws, causal=causal, mode=mode, out=out)
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    attn = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    return wall / steps * 1e3, prep, attn


def mode_peak(mode: str) -> float:
    return BF16_PEAK_TFLOPS if mode == "fp16" else FP4_PEAK_TFLOPS


def describe(name: str, c) -> str:
    return (f"{name}: B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} Sq=Skv={c['S']} D={c['D']} "
            f"causal={c['causal']} bf16 inputs")


def bench_attention(torch, mx, name, qt, kt, vt, modes, steps, warmup, min_warm_ms=0.0):
    """Every mode of one attention workload: whole step (K/V quantize +
    attention kernel) and the attention kernel alone, each against the peak
    of the mode's matrix-core type (FP4, or bf16 for the FP16 mode)."""
    c = dict(__import__("mxsynth").CONFIGS[name])
    flops = attn_flops(c)
    res = {"workload": describe(name, c), "flops": flops, "modes": {}}
    sha = kernel_source_sha()
    for mode in modes:
        ms, prep, attn = time_attention(torch, mx, qt, kt, vt, c, mode, steps, warmup, min_warm_ms)
        peak = mode_peak(mode)
        r = {"ms_per_step": ms, "tflops": flops / ms / 1e9, "prepare_ms": prep,
             "attn_kernel_ms": attn, "attn_kernel_tflops": flops / attn / 1e9,
             "attn_kernel_frac_peak": flops / attn / 1e9 / peak, "peak_tflops": peak,
             "steps": steps}
        if mode != "fp16":
            r["traffic"] = read_traffic(sha, f"{name}:{mode}")
        res["modes"][mode] = r
        log(f"[bench] {name} {mode}: {r}")
    return res


def read_traffic(sha: str, workload: str, kernel="attn_mx_kernel"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, if it was taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    entry = t.get(workload) if isinstance(t, dict) and "src_sha256" not in t else t
    if not isinstance(entry, dict) or entry.get("src_sha256") != sha:
        return None
    if entry.get("workload", workload) != workload:
        return None
    return entry.get("hbm_bytes_per_launch")


def bench_quantizer(torch, mx, reps=21, copies=3):
    """Quantize / dequantize the roundtrip tensor.  The timed loops rotate
    over ``copies`` distinct copies of it (flipped along rows: the same
    values at other addresses, 1.4 GB of input for three), so no pass finds
    its input in the 256 MB Infinity Cache left by the previous one."""
    import mxsynth
    log("[bench] quantizer: generating the 8192 x 28672 bf16 roundtrip tensor")
    x = mxsynth.roundtrip_tensor(2)
    x0 = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    del x
    xs = [x0] + [torch.flip(x0, dims=(0,)).contiguous() if i % 2 else x0.clone()
                 for i in range(1, copies)]
    n = x0.numel()
    codes = [torch.empty(n // 2, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    scales = [torch.empty(n // 32, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    ys = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    q_bytes = n * 2 + n // 2 + n // 32
    res = {"workload": "8192x28672 bf16, Student-t(3)*0.02 with 0.1% x50 outliers, blocks of 32 "
                       "along the last dim", "bytes_per_pass": q_bytes,
           "rotation": f"{copies} distinct input copies ({copies * n * 2 / 1e9:.2f} GB) taken in "
                       f"turn by the timed passes"}

    def timed(fn):
        warm(torch, lambda: [fn(i) for i in range(copies)])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for r in range(reps):
            fn(r % copies)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # streaming ceilings on the same tensors: a device-to-device copy (read
    # and write n bf16 elements) and a read-mostly pass (a max reduction)
    copy_ms = timed(lambda i: ys[i].copy_(xs[i].reshape(-1)))
    copy_gbps = 2 * n * 2 / copy_ms / 1e6
    red_ms = timed(lambda i: torch.amax(xs[i]))
    res["d2d_copy_ceiling"] = {"ms": copy_ms, "gbps": copy_gbps, "frac_hbm": copy_gbps / HBM_PEAK_GBPS}
    res["read_reduction"] = {"kernel": "torch.amax over the tensor (a library reduction, not a "
                                       "tuned streaming kernel: a lower bound on the read rate)",
                             "ms": red_ms,
                           "gbps": n * 2 / red_ms / 1e6, "frac_hbm": n * 2 / red_ms / 1e6 / HBM_PEAK_GBPS}
    for rule in ("uos", "ocp"):
        ms = timed(lambda i: mx.quantize(xs[i], rule, codes[i], scales[i]))
        mx.dequantize(codes[0], scales[0], out=ys[0])
        xf = x0.float().reshape(-1)
        err = (torch.linalg.vector_norm((xf - ys[0].float()).double()) /
               torch.linalg.vector_norm(xf.double())).item()
        res[rule] = {"quantize_ms": ms, "gbps": q_bytes / ms / 1e6,
                     "frac_hbm": q_bytes / ms / 1e6 / HBM_PEAK_GBPS,
                     "frac_copy_ceiling": q_bytes / ms / 1e6 / copy_gbps, "rel_frobenius": err}
        del xf
    ms = timed(lambda i: mx.dequantize(codes[i], scales[i], out=ys[i]))
    res["dequantize_bf16"] = {"ms": ms, "gbps": q_bytes / ms / 1e6,
                              "frac_hbm": q_bytes / ms / 1e6 / HBM_PEAK_GBPS,
                              "frac_copy_ceiling": q_bytes / ms / 1e6 / copy_gbps}
    return res


def bench_decode(torch, mx, reps=20, name="llm_decode", varlen=True):
    import mxsynth
    c = mxsynth.DECODE_CONFIGS[name]
    B, Hq, Hkv, Sq, Skv, D = c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Skv"], c["D"]
    log(f"[bench] decode: generating {name} inputs")
    q, k, v = mxsynth.llm_decode(c["seed"], B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D)
    to = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()  # noqa: E731
    qt, kt, vt = to(q), to(k), to(v)
    del q, k, v
    res = {"workload": f"{name}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} causal "
                       f"(end-aligned), bf16 inputs, KV cache quantized once",
           "split_keys": mx.decode_split(B, Hkv, Skv)}
    nt = (Skv + 127) // 128
    # one KV tile image: K codes (8 KiB), V codes (64 D), K and V scales (512 + 4 D),
    # rounded up to 1 KiB -- the quantized KV cache the kernel streams
    img_bytes = B * Hkv * nt * ((8192 + 64 * D + 512 + 4 * D + 1023) // 1024 * 1024)
    alg = img_bytes + B * Hq * Sq * D * 2 + B * Hq * Sq * D * 4  # KV cache, bf16 Q, fp32 O
    flops = 4.0 * B * Hq * Sq * Skv * D
    for mode in ("uos_pnq", "uos_efq"):
        ws = mx.alloc_decode_workspace(qt, kt, mode)
        mx.attn_prepare(qt, kt, vt, mode=mode, workspace=ws)
        out = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device="cuda")
        warm(torch, lambda: mx.attn_decode_prepared(qt, kt, ws, causal=True, mode=mode, out=out))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            mx.attn_decode_prepared(qt, kt, ws, causal=True, mode=mode, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[mode] = {"ms": ms, "gbps": alg / ms / 1e6, "frac_hbm": alg / ms / 1e6 / HBM_PEAK_GBPS,
                     "tflops": flops / ms / 1e9}
        del ws
    res["algorithmic_bytes"] = alg
    res["traffic"] = read_traffic(kernel_source_sha(ATTN_SOURCES), name, "attn_decode_kernel")
    if not varlen:
        return res

    # the same cache with per-entry lengths (mxattn_decode_varlen_prepared)
    vc = mxsynth.VARLEN_CONFIGS["llm_decode_varlen"]
    lens = mxsynth.seq_lengths(vc["lens_seed"], B, vc["lo"], vc["hi"])
    lk = torch.from_numpy(lens).cuda()
    vimg = int(sum(Hkv * ((int(n) + 127) // 128) * ((8192 + 64 * D + 512 + 4 * D + 1023) // 1024 * 1024)
                   for n in lens))
    valg = vimg + B * Hq * Sq * D * 2 + B * Hq * Sq * D * 4
    vflops = 4.0 * Hq * Sq * D * float(lens.sum())
    mode = "uos_pnq"
    ws = mx.alloc_decode_workspace(qt, kt, mode)
    mx.attn_prepare_varlen(qt, kt, vt, lk, mode=mode, workspace=ws)
    out = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device="cuda")
    warm(torch, lambda: mx.attn_decode_varlen_prepared(qt, kt, ws, lk, causal=True, mode=mode,
                                                        out=out))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        mx.attn_decode_varlen_prepared(qt, kt, ws, lk, causal=True, mode=mode, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    res["varlen"] = {"workload": f"llm_decode_varlen: the llm_decode cache with per-entry lengths "
                                 f"uniform on [{vc['lo']}, {vc['hi']}] (seed {vc['lens_seed']}): "
                                 f"{lens.tolist()}, {mode}",
                     "ms": ms, "algorithmic_bytes": valg, "gbps": valg / ms / 1e6,
                     "frac_hbm": valg / ms / 1e6 / HBM_PEAK_GBPS, "tflops": vflops / ms / 1e9}
    del ws
    return res


def bench_prefill_varlen(torch, mx, reps=5, name="llm_prefill_varlen"):
    """The LLM prefill batch (B=4, 32/8 heads, D=128, causal) with per-entry
    prompt lengths, one mxattn_fwd_varlen call (K/V quantize + attention)
    per step; flops count only each entry's own causal pairs."""
    import mxsynth
    vc = mxsynth.VARLEN_CONFIGS[name]
    c = mxsynth.CONFIGS[vc["base"]]
    B, Hq, S, D = c["B"], c["Hq"], c["S"], c["D"]
    log(f"[bench] prefill varlen: generating {vc['base']} inputs")
    q, k, v = mxsynth.make_attn_inputs(vc["base"])
    to = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()  # noqa: E731
    qt, kt, vt = to(q), to(k), to(v)
    del q, k, v
    lens = mxsynth.seq_lengths(vc["lens_seed"], B, vc["lo"], vc["hi"])
    lt = torch.from_numpy(lens).cuda()
    flops = sum(4.0 * Hq * D * int(n) * (int(n) + 1) / 2 for n in lens)
    mode = "uos_pnq"
    ws = mx.alloc_workspace(qt, kt, mode)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    warm(torch, lambda: mx.attn_fwd_varlen(qt, kt, vt, lt, lt, causal=True, mode=mode, out=out,
                                           workspace=ws))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        mx.attn_fwd_varlen(qt, kt, vt, lt, lt, causal=True, mode=mode, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"workload": f"{name}: {vc['base']} (B={B} Hq={Hq} Hkv={c['Hkv']} S<={S} D={D} causal, "
                        f"bf16) with per-entry lengths uniform on [{vc['lo']}, {vc['hi']}] "
                        f"(seed {vc['lens_seed']}): {lens.tolist()}, {mode}",
            "ms": ms, "flops": flops, "tflops": flops / ms / 1e9,
            "frac_fp4_peak": flops / ms / 1e9 / FP4_PEAK_TFLOPS}


def library_scaled_mm(torch, xc, xs, wc, ws, M, N, K, y, timed):
    """The same MXFP4 operands (codes two E2M1 per byte, low nibble first;
    E8M0 bytes per 32 along K) through torch's block-scaled matrix product
    (hipBLASLt on this GPU), for comparison only: its time and its largest
    difference from this library's bf16 output."""
    # the library call takes whole 128-row blocks: a is padded with zero rows
    Mp = (M + 127) // 128 * 128
    ap = torch.zeros((Mp, K // 2), dtype=torch.uint8, device=xc.device)
    ap[:M] = xc.view(M, K // 2)
    sp = torch.full((Mp, K // 32), 127, dtype=torch.uint8, device=xc.device)
    sp[:M] = xs.view(M, K // 32)
    a4 = ap.view(torch.float4_e2m1fn_x2)
    b4 = wc.view(N, K // 2).view(torch.float4_e2m1fn_x2)
    sa = sp.view(torch.float8_e8m0fnu)
    sb = ws.view(N, K // 32).view(torch.float8_e8m0fnu)
    try:
        r = torch._scaled_mm(a4, b4.t(), sa, sb, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
    except Exception as e:  # an unsupported shape or build: reported, not fatal
        return {"error": repr(e)[:300]}
    diff = (r[:M].float() - y.float()).abs().max().item()
    ymax = y.float().abs().max().item()
    del r
    ms = timed(lambda: torch._scaled_mm(a4, b4.t(), sa, sb, out_dtype=torch.bfloat16))
    return {"call": "torch._scaled_mm (float4_e2m1fn_x2 operands, float8_e8m0fnu scales, bf16 out)",
            "rows": Mp, "ms": ms, "tflops": 2.0 * Mp * N * K / ms / 1e9,
            "max_abs_diff_vs_library": diff, "max_abs_output": ymax}


def library_attention(torch, qt, kt, vt, c, steps):
    """torch's fused bf16 attention (the flash backend only, so that no
    unfused fallback runs) on the same bf16 q, k, v, for comparison only."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    G = c["Hq"] // c["Hkv"]
    kk = kt if G == 1 else kt.repeat_interleave(G, dim=1).contiguous()
    vv = vt if G == 1 else vt.repeat_interleave(G, dim=1).contiguous()
    fn = lambda: F.scaled_dot_product_attention(qt, kk, vv, is_causal=bool(c["causal"]))  # noqa: E731
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            o = fn()
            torch.cuda.synchronize()
            finite = bool(torch.isfinite(o).all().item())
            del o
            warm(torch, fn)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
    except Exception as e:  # no fused kernel for this build or shape: reported, not fatal
        return {"error": repr(e)[:300]}
    ms = e0.elapsed_time(e1) / steps
    f = attn_flops(c)
    return {"call": "torch.nn.functional.scaled_dot_product_attention, flash backend, bf16",
            "ms": ms, "tflops": f / ms / 1e9, "frac_bf16_peak": f / ms / 1e9 / BF16_PEAK_TFLOPS,
            "finite": finite}


def bench_gemm(torch, mx, reps=10, name="dit14_ffn_up", library=False):
    import mxsynth
    g = mxsynth.GEMM_CONFIGS[name]
    M, N, K = g["M"], g["N"], g["K"]
    log(f"[bench] gemm: generating {name} operands")
    x, w = mxsynth.make_gemm_inputs(name)
    to = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()  # noqa: E731
    xt, wt = to(x), to(w)
    del x, w
    wc, ws = mx.quantize(wt, "uos")   # the weight is quantized once, ahead of time
    xc = torch.empty(M * K // 2, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M * K // 32, dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * M * N * K

    def timed(fn):
        warm(torch, fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    work = mx.gemm_workspace(M, N, K)
    mx.quantize(xt, "uos", xc, xs)
    gemm_ms = timed(lambda: mx.gemm(xc, xs, wc, ws, M, N, K, out=y, workspace=work))
    lin_ms = timed(lambda: (mx.quantize(xt, "uos", xc, xs),
                            mx.gemm(xc, xs, wc, ws, M, N, K, out=y, workspace=work)))
    alg_bytes = M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + M * N * 2
    res = {"workload": f"{name}: x [{M}, {K}] bf16 (N(0,1), 1% channels x20) times UOS-MXFP4 "
                       f"weight [{N}, {K}] (Student-t(3)*0.02, 0.1% x50), bf16 output",
           "flops": flops, "algorithmic_bytes": alg_bytes,
           "traffic": read_traffic(kernel_source_sha(GEMM_SOURCES), name, "gemm_mx_kernel"),
           "gemm_ms": gemm_ms, "gemm_tflops": flops / gemm_ms / 1e9,
           "gemm_frac_fp4_peak": flops / gemm_ms / 1e9 / FP4_PEAK_TFLOPS,
           "linear_w4a4_ms": lin_ms, "linear_w4a4_tflops": flops / lin_ms / 1e9}
    if library:
        mx.gemm(xc, xs, wc, ws, M, N, K, out=y, workspace=work)
        res["library_scaled_mm"] = library_scaled_mm(torch, xc, xs, wc, ws, M, N, K, y, timed)
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Query rows per head of the oracle sample: about 10-30 s of host work.
CPU_ROWS_PER_HEAD = {"dit13": 1024, "dit14": 2048, "llm_prefill": 1024}


def cpu_baseline(q, k, v, c, name):
    """The oracle (as it stands) on a bounded, seeded sample of query rows of
    every head of the workload, against all keys."""
    import mxsynth
    import oracle
    rows_per_head = CPU_ROWS_PER_HEAD[name]
    rows = mxsynth.sample_rows(c["seed"], c["B"], c["Hq"], c["S"], rows_per_head)
    t0 = time.perf_counter()
    oracle.attn_rows(q, k, v, causal=c["causal"], mode=oracle.MODE_UOS_PNQ, bc=128, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * rows.size * c["S"] * c["D"] * (0.5 if c["causal"] else 1.0)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": dt,
            # an extrapolation, not a measurement: the whole workload at the
            # sample's rate
            "full_problem_seconds_extrapolated": attn_flops(c) / (flops / dt),
            "sample": f"{name} UOS+PNQ, {rows.size} seeded query rows ({rows_per_head} from each "
                      f"of the {c['B'] * c['Hq']} heads) against all {c['S']} keys, binary64, "
                      f"including the K/V quantization of those heads"}


# Modes timed per attention workload (the first is the headline when the
# workload is the headline one).
WORKLOAD_MODES = {
    "dit13": ("uos_pnq", "fp16", "ocp", "uos_efq"),
    "dit14": ("uos_pnq", "uos_efq", "fp16", "ocp", "uos"),
    "llm_prefill": ("uos_pnq", "uos_efq", "ocp", "uos"),
}
SECTION_STEPS = {"dit13": 5, "dit14": 10, "llm_prefill": 20}


def load_inputs(torch, name):
    import mxsynth
    log(f"[bench] generating {name} inputs")
    q, k, v = mxsynth.make_attn_inputs(name)
    to = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()  # noqa: E731
    return (q, k, v), (to(q), to(k), to(v))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit13", choices=sorted(WORKLOAD_MODES))
    ap.add_argument("--modes", default=None,
                    help="comma list; the first is the headline, the rest run alongside "
                         "(default: every mode of the workload, UOS+PNQ first)")
    ap.add_argument("--sections", default="dit14,llm_prefill",
                    help="other attention workloads timed in every mode ('' for none)")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the per-sequence-length sections (prefill, decode)")
    ap.add_argument("--no-attention", action="store_true",
                    help="only the standalone quantizer, the GEMM and the decode sections "
                         "(for profiling them alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--library-attention", action="store_true",
                    help="also time torch's fused bf16 attention on the headline workload "
                         "(a comparison, off by default)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch's block-scaled MXFP4 matrix product on the same "
                         "GEMM operands (a comparison, off by default)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import mxfp4_block_quantized_amd as mx
    import mxsynth

    mx.lib()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    if args.no_attention:
        res = {}
        if not args.no_quantizer:
            res["quantizer"] = bench_quantizer(torch, mx, reps=3)
        if not args.no_gemm:
            res["gemm"] = bench_gemm(torch, mx, reps=3, library=args.library_gemm)
        if not args.no_decode:
            res["decode"] = bench_decode(torch, mx, reps=20, varlen=not args.no_varlen)
        print(json.dumps(res), flush=True)
        return

    c = dict(mxsynth.CONFIGS[args.workload])
    host, (qt, kt, vt) = load_inputs(torch, args.workload)
    modes = args.modes.split(",") if args.modes else list(WORKLOAD_MODES[args.workload])
    head = modes[0]
    # the headline mode: --warmup untimed steps, then exactly --steps timed
    # steps; the modes alongside: half as many
    headline = bench_attention(torch, mx, args.workload, qt, kt, vt, [head], args.steps,
                               args.warmup)
    along = bench_attention(torch, mx, args.workload, qt, kt, vt, modes[1:],
                            max(3, args.steps // 2), max(1, args.warmup // 2)) if modes[1:] else None
    library = library_attention(torch, qt, kt, vt, c, max(3, args.steps // 2)) \
        if args.library_attention else None
    del qt, kt, vt
    torch.cuda.empty_cache()
    hr = headline["modes"][head]
    flops = headline["flops"]
    peak = mode_peak(head)
    roofline = {"bound": "mfma", "kernel": "attn_mx_kernel" if head != "fp16" else "attn_f16_kernel",
                "achieved": hr["attn_kernel_tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": hr["attn_kernel_tflops"] / peak,
                "traffic": hr.get("traffic"),
                "algorithmic_flops_per_launch": flops,
                "launch_ms": hr["attn_kernel_ms"]}
    out = {
        "metric": METRIC,
        "value": hr["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": hr["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if head != "fp16" else "bf16/fp16",
        "data": "synthetic",
        "config": {"workload": f"{describe(args.workload, c)}, mode {head}",
                   "B": c["B"], "Hq": c["Hq"], "Hkv": c["Hkv"], "S": c["S"], "D": c["D"],
                   "causal": c["causal"], "mode": head, "kv_tile": mx.kv_tile(c["D"], head)},
        "pct_fp4_peak": 100.0 * hr["tflops"] / FP4_PEAK_TFLOPS,
        "roofline": roofline,
        "alongside": along["modes"] if along else {},
    }
    if library is not None:
        out["library_attention"] = library
    sections = [w for w in args.sections.split(",") if w and w != args.workload]
    if sections:
        out["attention"] = {}
    for name in sections:
        _, (sq, sk, sv) = load_inputs(torch, name)
        out["attention"][name] = bench_attention(torch, mx, name, sq, sk, sv,
                                                 list(WORKLOAD_MODES[name]),
                                                 SECTION_STEPS.get(name, 5), 3, min_warm_ms=200.0)
        del sq, sk, sv
        torch.cuda.empty_cache()
    if not args.no_quantizer:
        out["quantizer"] = bench_quantizer(torch, mx)
        log(f"[bench] quantizer: {out['quantizer']}")
    if not args.no_gemm:
        out["gemm"] = bench_gemm(torch, mx, library=args.library_gemm)
        log(f"[bench] gemm: {out['gemm']}")
    if not args.no_decode:
        out["decode"] = bench_decode(torch, mx, varlen=not args.no_varlen)
        log(f"[bench] decode: {out['decode']}")
    if not args.no_varlen:
        out["prefill_varlen"] = bench_prefill_varlen(torch, mx)
        log(f"[bench] prefill varlen: {out['prefill_varlen']}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle sample)")
        q, k, v = host
        out["cpu_baseline"] = cpu_baseline(q, k, v, c, args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
