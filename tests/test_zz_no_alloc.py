"""mxgemm_noalloc (the W4A4 product with the library's own scratch instead of
a caller workspace) against mxgemm, called through the C ABI: two calls in a
row, the second smaller, each bit-identical to mxgemm on the same operands
(the same kernels run; only where the E8M0 staging lives differs).  Also:
shapes whose staging exceeds the scratch are refused before any launch."""
import ctypes

import numpy as np
import pytest

from common import gpu, mxsynth, to_torch

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20


def _operands(torch, mx, seed, M, N, K, rule):
    x, w = mxsynth.w4a4_operands(seed, M, N, K)
    ac, asc = mx.quantize(to_torch(x), rule)
    bc, bsc = mx.quantize(to_torch(w), rule)
    return ac, asc, bc, bsc


def _noalloc(torch, mx, ac, asc, bc, bsc, M, N, K, out):
    L = mx.lib()
    s = torch.cuda.current_stream()
    st = L.mxgemm_noalloc(ctypes.c_void_p(ac.data_ptr()), ctypes.c_void_p(asc.data_ptr()),
                          ctypes.c_void_p(bc.data_ptr()), ctypes.c_void_p(bsc.data_ptr()),
                          M, N, K, 1 if out.dtype == torch.bfloat16 else 0,
                          ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
    assert st == 0, L.mx_strerror(st)
    return out


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry(out_dtype):
    torch, mx = gpu()
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    # a large call, then a smaller one: the scratch keeps the first call's
    # staging, which the second must not read
    cases = [(2100, 1500, 4608, 71, "uos"), (300, 260, 1024, 72, "ocp")]
    for M, N, K, seed, rule in cases:
        assert mx.lib().mxgemm_workspace_bytes(M, N, K) <= SCRATCH
        ac, asc, bc, bsc = _operands(torch, mx, seed, M, N, K, rule)
        want = mx.gemm(ac, asc, bc, bsc, M, N, K, out_dtype=dt)
        got = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
        _noalloc(torch, mx, ac, asc, bc, bsc, M, N, K, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (M, N, K)
        print(f"noalloc M={M} N={N} K={K} {rule} {out_dtype}: identical to mxgemm")


def test_noalloc_full_dit_shape_and_limit():
    torch, mx = gpu()
    # the feed-forward up-projection of the DiT (the bench's GEMM shape)
    M, N, K = 32760, 13824, 5120
    ac, asc, bc, bsc = _operands(torch, mx, 6, M, N, K, "uos")
    want = mx.gemm(ac, asc, bc, bsc, M, N, K, out_dtype=torch.bfloat16)
    got = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _noalloc(torch, mx, ac, asc, bc, bsc, M, N, K, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # staging past the scratch: refused (no launch, nothing written)
    L = mx.lib()
    Kbig = 23040 + 128
    assert L.mxgemm_workspace_bytes(M, N, Kbig) > SCRATCH
    P = ctypes.c_void_p(ac.data_ptr())
    assert L.mxgemm_noalloc(P, P, P, P, M, N, Kbig, 1, ctypes.c_void_p(got.data_ptr()),
                            None) == -2
    assert torch.equal(got, want)
