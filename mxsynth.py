"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no quantization or attention arithmetic: it only draws
random tensors with the shapes and value distributions of the workloads and
stores them in their working dtype.  Every generator takes a seed and draws
from ``numpy.random.default_rng(seed)`` in a fixed, documented order, so the
GPU path and the CPU oracle always see the same bits.

bf16 tensors are returned as their raw bit patterns (``uint16``), rounded
from float32 to nearest-even.  The workloads stand in for the video
diffusion and LLM attention layers named on the MXAttention and EFQ-Softmax
pages (no model, checkpoint or benchmark suite is used).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "tiny_attn", "tiny_quant",
    "roundtrip_tensor", "llm_prefill", "video_dit", "sample_rows", "CONFIGS",
    "w4a4_operands", "GEMM_CONFIGS", "make_gemm_inputs", "llm_decode", "DECODE_CONFIGS",
]


def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.
    Inputs are finite."""
    x = np.ascontiguousarray(x, np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.size, np.uint16)
    for s in range(0, flat.size, chunk):
        u = flat[s:s + chunk].view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out[s:s + chunk] = r.astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def tiny_attn(seed: int = 0, S: int = 256, D: int = 64):
    """q, k, v [1, 1, S, D] float32, i.i.d. N(0, 1), drawn q then k then v."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (1, 1, S, D))
    k = _normal(rng, (1, 1, S, D))
    v = _normal(rng, (1, 1, S, D))
    return q, k, v


def tiny_quant(seed: int = 1, nblocks: int = 4096):
    """[nblocks, 32] float32: the first half of the blocks N(0, 1), the
    second half Student-t with 3 degrees of freedom."""
    rng = np.random.default_rng(seed)
    half = nblocks // 2
    a = _normal(rng, (half, 32))
    b = rng.standard_t(3, size=(nblocks - half, 32)).astype(np.float32)
    return np.concatenate([a, b], axis=0)


def roundtrip_tensor(seed: int = 2, rows: int = 8192, cols: int = 28672):
    """[rows, cols] bf16 bits: Student-t(3) * 0.02, with a Bernoulli(0.001)
    mask of entries multiplied by 50 (outliers).  Drawn in row chunks."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), np.uint16)
    step = max(1, (1 << 23) // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        t = rng.standard_t(3, size=(r1 - r0, cols)).astype(np.float32) * np.float32(0.02)
        mask = rng.random(size=(r1 - r0, cols), dtype=np.float32) < np.float32(0.001)
        t[mask] *= np.float32(50.0)
        out[r0:r1] = f32_to_bf16_bits(t)
    return out


def llm_prefill(seed: int = 3, B: int = 4, Hq: int = 32, Hkv: int = 8,
                S: int = 8192, D: int = 128, frac: float = 0.02, gain: float = 15.0):
    """Causal GQA prefill shapes.  q [B,Hq,S,D], k/v [B,Hkv,S,D], bf16 bits.

    Draw order: q, k, v ~ N(0,1); then for each KV head g in order,
    round(frac*D) distinct channels (``rng.choice``) multiplied by ``gain``
    in K head g and in the query heads that read it."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, Hq, S, D))
    k = _normal(rng, (B, Hkv, S, D))
    v = _normal(rng, (B, Hkv, S, D))
    nch = int(round(frac * D))
    group = Hq // Hkv
    for g in range(Hkv):
        ch = rng.choice(D, nch, replace=False)
        k[:, g, :, ch] *= np.float32(gain)
        for h in range(g * group, (g + 1) * group):
            q[:, h, :, ch] *= np.float32(gain)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def llm_decode(seed: int = 8, B: int = 8, Hq: int = 32, Hkv: int = 8, Sq: int = 1,
               Skv: int = 32768, D: int = 128, frac: float = 0.02, gain: float = 15.0):
    """Short-query GQA shapes (a decode step against a long key/value cache):
    q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D], bf16 bits.  The recipe of
    ``llm_prefill`` with separate query and key lengths: q, k, v ~ N(0,1) in
    that order (k and v in chunks of KV heads), then per KV head round(frac*D)
    channels (``rng.choice``) x gain in K head g and its query heads."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, Hq, Sq, D))
    k = np.empty((B, Hkv, Skv, D), np.uint16)
    v = np.empty((B, Hkv, Skv, D), np.uint16)
    nch = int(round(frac * D))
    group = Hq // Hkv
    chans = []
    kf = [_normal(rng, (B, 1, Skv, D)) for _ in range(Hkv)]
    for g in range(Hkv):
        v[:, g:g + 1] = f32_to_bf16_bits(_normal(rng, (B, 1, Skv, D)))
    for g in range(Hkv):
        ch = rng.choice(D, nch, replace=False)
        chans.append(ch)
        kf[g][:, :, :, ch] *= np.float32(gain)
        k[:, g:g + 1] = f32_to_bf16_bits(kf[g])
        kf[g] = None
        for h in range(g * group, (g + 1) * group):
            q[:, h, :, ch] *= np.float32(gain)
    return f32_to_bf16_bits(q), k, v


def _smooth_bias(rng, grid, std):
    """N(0,1) on the latent grid, 3x5x5 box filter (reflecting edges),
    renormalised to unit std, times ``std``; flattened token order
    t = (f*H + y)*W + x."""
    from scipy.ndimage import uniform_filter
    z = rng.standard_normal(size=grid)
    z = uniform_filter(z, size=(3, 5, 5), mode="reflect")
    z = (z - z.mean()) / z.std()
    return (z * std).reshape(-1).astype(np.float32)


def video_dit(seed: int = 4, H: int = 40, grid=(21, 30, 52), D: int = 128,
              frac: float = 0.01, gain: float = 20.0, bias_std: float = 0.5):
    """Video-DiT self-attention shapes, B = 1, S = prod(grid), bf16 bits.

    Draw order: q, k, v ~ N(0,1) [1,H,S,D]; per head h in order,
    round(frac*D) channels (``rng.choice``) multiplied by ``gain`` in both
    q and k of that head; then a smooth per-token bias for q and then one
    for k (std ``bias_std``), added to every channel of every head."""
    rng = np.random.default_rng(seed)
    S = int(np.prod(grid))
    q = _normal(rng, (1, H, S, D))
    k = _normal(rng, (1, H, S, D))
    v = _normal(rng, (1, H, S, D))
    nch = max(1, int(round(frac * D)))
    for h in range(H):
        ch = rng.choice(D, nch, replace=False)
        q[:, h, :, ch] *= np.float32(gain)
        k[:, h, :, ch] *= np.float32(gain)
    bq = _smooth_bias(rng, grid, bias_std)
    bk = _smooth_bias(rng, grid, bias_std)
    for h in range(H):
        q[0, h] += bq[:, None]
        k[0, h] += bk[:, None]
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def sample_rows(seed: int, B: int, H: int, S: int, n: int = 256) -> np.ndarray:
    """Flattened query-row indices (b*H + h)*S + i: ``n`` distinct rows per
    (b, h), drawn in (b, h) order from ``default_rng(seed + 100)``.  If
    n >= S every row is returned."""
    if n >= S:
        return np.arange(B * H * S, dtype=np.int64)
    rng = np.random.default_rng(seed + 100)
    out = []
    for bh in range(B * H):
        idx = np.sort(rng.choice(S, n, replace=False))
        out.append(bh * S + idx)
    return np.concatenate(out).astype(np.int64)


# Workload table: name -> attention shape and generator.
CONFIGS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, S=256, D=64, causal=False, seed=0,
                 dtype="f32", modes=("fp16", "ocp", "uos", "uos_pnq")),
    "llm_prefill": dict(B=4, Hq=32, Hkv=8, S=8192, D=128, causal=True, seed=3,
                        dtype="bf16", modes=("ocp", "uos", "uos_pnq")),
    "dit14": dict(B=1, Hq=40, Hkv=40, S=32760, D=128, causal=False, seed=4,
                  dtype="bf16", grid=(21, 30, 52),
                  modes=("fp16", "ocp", "uos", "uos_pnq")),
    "dit13": dict(B=1, Hq=24, Hkv=24, S=118800, D=128, causal=False, seed=5,
                  dtype="bf16", grid=(33, 45, 80), modes=("fp16", "uos_pnq")),
}


def make_attn_inputs(name: str):
    """(q, k, v) for a named workload of ``CONFIGS``."""
    c = CONFIGS[name]
    if name == "tiny":
        return tiny_attn(c["seed"], c["S"], c["D"])
    if name == "llm_prefill":
        return llm_prefill(c["seed"], c["B"], c["Hq"], c["Hkv"], c["S"], c["D"])
    return video_dit(c["seed"], c["Hq"], c["grid"], c["D"])


def w4a4_operands(seed: int, M: int, N: int, K: int):
    """Operands of a linear layer of the video DiT: activations x [M, K] (one
    row per latent token) and weight w [N, K] (one row per output feature),
    bf16 bits.  x is N(0, 1) with round(0.01 K) outlier channels, chosen
    with ``rng.choice(K, n, replace=False)``, scaled by 20 (the outlier
    recipe of the attention inputs); w is Student-t(3) * 0.02 with a
    Bernoulli(0.001) mask of entries scaled by 50 (the roundtrip tensor's
    recipe).  Draw order: outlier channels, x in row chunks, w in row chunks."""
    rng = np.random.default_rng(seed)
    ch = rng.choice(K, max(1, round(0.01 * K)), replace=False)
    gain = np.ones(K, np.float32)
    gain[ch] = 20.0
    x = np.empty((M, K), np.uint16)
    step = max(1, (1 << 23) // K)
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        x[r0:r1] = f32_to_bf16_bits(_normal(rng, (r1 - r0, K)) * gain)
    w = np.empty((N, K), np.uint16)
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        t = rng.standard_t(3, size=(r1 - r0, K)).astype(np.float32) * np.float32(0.02)
        mask = rng.random(size=(r1 - r0, K), dtype=np.float32) < np.float32(0.001)
        t[mask] *= np.float32(50.0)
        w[r0:r1] = f32_to_bf16_bits(t)
    return x, w


# Linear layers of the video DiT (hidden 5120 = 40 heads x 128, feed-forward
# 13824) over the 32760 latent tokens of the dit14 attention workload.
GEMM_CONFIGS = {
    "dit14_ffn_up": dict(M=32760, N=13824, K=5120, seed=6),
    "dit14_ffn_down": dict(M=32760, N=5120, K=13824, seed=7),
}


def make_gemm_inputs(name: str):
    """(x, w) for a named workload of ``GEMM_CONFIGS``."""
    c = GEMM_CONFIGS[name]
    return w4a4_operands(c["seed"], c["M"], c["N"], c["K"])


# Short-query workloads: one decode step of the LLM shape (32 query heads,
# 8 KV heads, D = 128) against a 32K-token cache.
DECODE_CONFIGS = {
    "llm_decode": dict(B=8, Hq=32, Hkv=8, Sq=1, Skv=32768, D=128, causal=True, seed=8),
}


# Padded batches of sequences with their own lengths: the LLM prefill batch
# with per-entry prompt lengths (causal self-attention, query length = key
# length) and the decode batch with per-entry KV-cache lengths.
VARLEN_CONFIGS = {
    "llm_prefill_varlen": dict(base="llm_prefill", lens_seed=10, lo=512, hi=8192),
    "llm_decode_varlen": dict(base="llm_decode", lens_seed=11, lo=1024, hi=32768),
}


def seq_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-entry lengths of a padded batch: B integers uniform on [lo, hi]
    (``rng.integers``), int32."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)
