"""GPU parity of the W4A4 product (``mxgemm``) against the binary64 oracle.

Bar: the MXFP4 products are exact and the kernel adds them in fp32, one
128-element matrix instruction at a time, so |y - y_oracle| <=
(K/128 + 2) * 2^-24 * sum_k |a_k b_k| for fp32 output; a bf16 output adds
its own rounding, 2^-8 |y| at most (half an ulp is 2^-9 relative, doubled
for the fp32 error underneath).  Quantized operands fed to the kernel come
from the oracle (small cases) or from the GPU quantizer after a bit-exact
check against the oracle (full sizes).
"""
import functools

import numpy as np
import pytest

from common import gpu, mxsynth, np_u8, oracle, to_torch

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def bound(K, yabs, y, bf16):
    b = (K / 128 + 2) * U32 * yabs
    if bf16:
        b = b * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y)
    return b + 1e-37


def check(got, y, yabs, K, bf16, label):
    err = np.abs(got - y)
    b = bound(K, yabs, y, bf16)
    ratio = float((err / b).max())
    print(f"[gemm] {label}: max|err| {err.max():.3e}  max err/bound {ratio:.3f}  "
          f"max|y| {np.abs(y).max():.3e}", flush=True)
    assert np.all(err <= b), label


def torch_out(torch, y):
    return y.float().cpu().numpy().astype(np.float64)


def run_small(M, N, K, rule, out_bf16, seed, scale=1.0):
    torch, mx = gpu()
    print(f"[case] gemm M={M} N={N} K={K} rule={rule} bf16={out_bf16}", flush=True)
    rng = np.random.default_rng(seed)
    a = (rng.standard_t(3, (M, K)) * scale).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    y, yabs, (ac, as_), (bc, bs) = oracle.gemm(a, b, rule)
    dev = lambda t: torch.from_numpy(t).cuda()
    out = mx.gemm(dev(ac), dev(as_), dev(bc), dev(bs), M, N, K,
                  out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    check(torch_out(torch, out), y, yabs, K, out_bf16, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("shape", [(1, 1, 128), (5, 7, 256), (300, 200, 384), (256, 256, 128),
                                   (513, 777, 1024), (1000, 260, 640), (64, 1030, 2048)])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_small_shapes(shape, out_bf16):
    M, N, K = shape
    run_small(M, N, K, oracle.RULE_UOS, out_bf16, seed=7 * M + 3 * N + K)


@pytest.mark.parametrize("rule", [oracle.RULE_OCP, oracle.RULE_UOS])
def test_rules_and_wide_range(rule):
    # rows of very different magnitude: per-block scales must reach the matrix core
    run_small(384, 300, 512, rule, False, seed=70, scale=2.0 ** 20)
    run_small(384, 300, 512, rule, False, seed=71, scale=2.0 ** -30)


def test_odd_n_scalar_stores():
    run_small(300, 203, 256, oracle.RULE_UOS, False, seed=72)
    run_small(300, 203, 256, oracle.RULE_UOS, True, seed=73)


def test_zero_operand_gives_zero():
    torch, mx = gpu()
    M, N, K = 300, 500, 384
    ac = torch.zeros(M * K // 2, dtype=torch.uint8, device="cuda")
    as_ = torch.zeros(M * K // 32, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(74)
    b = rng.standard_normal((N, K)).astype(np.float32)
    bc, bs = oracle.quantize(b, oracle.RULE_UOS)
    out = mx.gemm(ac, as_, torch.from_numpy(bc).cuda(), torch.from_numpy(bs).cuda(), M, N, K)
    assert torch.count_nonzero(out).item() == 0


def test_deterministic_and_linear_w4a4():
    torch, mx = gpu()
    M, N, K = 700, 600, 1024
    x, w = mxsynth.w4a4_operands(75, M, N, K)
    xt, wt = to_torch(x), to_torch(w)
    wc, ws = mx.quantize(wt, "uos")
    y1 = mx.linear_w4a4(xt, wc, ws, N, "uos", out_dtype=torch.float32)
    y2 = mx.linear_w4a4(xt, wc, ws, N, "uos", out_dtype=torch.float32)
    assert torch.equal(y1, y2)
    y, yabs, _, _ = oracle.gemm(x, w, oracle.RULE_UOS)
    check(torch_out(torch, y1), y, yabs, K, False, "linear_w4a4 700x600x1024")


@pytest.mark.parametrize("shape", [(4352, 4352, 640), (4352, 4400, 512), (4500, 4352, 1536)])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_many_tiles_per_workgroup(shape, out_bf16):
    """More output tiles than compute units: each workgroup walks several
    tiles (odd and even numbers of 256-K stages, full and ragged tiles)."""
    torch, mx = gpu()
    M, N, K = shape
    print(f"[case] gemm many tiles M={M} N={N} K={K} bf16={out_bf16}", flush=True)
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    ac, as_ = oracle.quantize(a, oracle.RULE_UOS)
    bc, bs = oracle.quantize(b, oracle.RULE_UOS)
    dev = lambda t: torch.from_numpy(t).cuda()
    out = mx.gemm(dev(ac), dev(as_), dev(bc), dev(bs), M, N, K,
                  out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    rows = np.sort(rng.choice(M, 96, replace=False))
    rows[-1] = M - 1
    y, yabs = oracle.gemm_q(ac.reshape(M, K // 2)[rows], as_.reshape(M, K // 32)[rows], bc, bs,
                            rows.size, N, K)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    check(got, y, yabs, K, out_bf16, f"many tiles {shape}")


# ----------------------------------------------------------- full sizes ----

@functools.lru_cache(maxsize=1)
def full_inputs(name):
    return mxsynth.make_gemm_inputs(name)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dit14_ffn_up", "dit14_ffn_down"])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_full_dit14_linear(name, out_bf16):
    torch, mx = gpu()
    c = mxsynth.GEMM_CONFIGS[name]
    M, N, K = c["M"], c["N"], c["K"]
    print(f"[case] {name} M={M} N={N} K={K} bf16={out_bf16}", flush=True)
    x, w = full_inputs(name)
    xt, wt = to_torch(x), to_torch(w)
    xc, xs = mx.quantize(xt, "uos")
    wc, ws = mx.quantize(wt, "uos")
    out = mx.gemm(xc, xs, wc, ws, M, N, K, out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(c["seed"] + 100).choice(M, 256, replace=False))
    # the GPU quantizer's codes of the weight and of the sampled rows are the oracle's
    owc, ows = oracle.quantize(w, oracle.RULE_UOS)
    assert np.array_equal(np_u8(wc), owc) and np.array_equal(np_u8(ws), ows)
    oxc, oxs = oracle.quantize(x[rows], oracle.RULE_UOS)
    gxc = np_u8(xc).reshape(M, K // 2)[rows]
    gxs = np_u8(xs).reshape(M, K // 32)[rows]
    assert np.array_equal(gxc.reshape(-1), oxc) and np.array_equal(gxs.reshape(-1), oxs)
    y, yabs = oracle.gemm_q(gxc, gxs, owc, ows, rows.size, N, K)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    check(got, y, yabs, K, out_bf16, f"{name} (256 sampled rows)")
