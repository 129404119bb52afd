"""CPU oracle for MXFP4 block quantization and MXFP4 attention.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``mxfp4_block_quantized_amd``) never imports it, and it never imports the GPU
library; the two share no code.

The arithmetic lives in ``mxoracle.c`` (plain C, binary64, OpenMP over rows and
blocks).  This module only builds it with gcc and marshals numpy arrays.
What each function computes, with its sources, is documented in the C file:

* the OCP scale rule and Universal Optimal Scaling (boundary 7.25) --
  "MXAttention: Data-Free Optimal Scaling and Pre-Normalization Quantization
  for MXFP4 Attention", abstract;
* rounding onto the eight E2M1 magnitudes with an exact power-of-two scale --
  "Quantization Error", section "Where the error comes from";
* the online-softmax loop with one quantized probability operand feeding both
  numerator and denominator -- "EFQ-Softmax", abstract, and the PNQ component
  of the MXAttention abstract;
* the W4A4 product of two MXFP4 operands quantized along the contraction
  ("MXCode", abstract: MX-native W4A4 operands), here in numpy: the
  operands are decoded by ``dequantize`` and multiplied in binary64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")

F32, BF16 = 0, 1
RULE_OCP, RULE_UOS = 0, 1
MODE_FP16, MODE_OCP, MODE_UOS, MODE_UOS_PNQ, MODE_UOS_EFQ = 0, 1, 2, 3, 4
BLOCK = 32

_lib = None


def build(force: bool = True) -> str:
    """Compile ``mxoracle.c`` into ``_liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        cmd = [
            "gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            _SRC, "-o", _LIB + ".tmp", "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_scale_exponent.argtypes = [ctypes.c_double, ci]
    lib.oracle_scale_exponent.restype = ci
    lib.oracle_round_e2m1.argtypes = [ctypes.c_double]
    lib.oracle_round_e2m1.restype = ci
    lib.oracle_quantize.argtypes = [P, ci, i64, ci, P, P]
    lib.oracle_quantize.restype = ci
    lib.oracle_quantize_t.argtypes = [P, ci, i64, i64, ci, P, P]
    lib.oracle_quantize_t.restype = ci
    lib.oracle_dequantize.argtypes = [P, P, i64, P]
    lib.oracle_dequantize.restype = ci
    lib.oracle_attn_rows.argtypes = [P, P, P, ci] + [ci] * 9 + [P, i64, P, P, P, P, P, P]
    lib.oracle_attn_rows.restype = ci
    lib.oracle_attn_rows_split.argtypes = [P, P, P, ci] + [ci] * 9 + [i64, P, i64, P, P, P, P, P, P]
    lib.oracle_attn_rows_split.restype = ci
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ci
    lib.oracle_efq_beta.argtypes = []
    lib.oracle_efq_beta.restype = ctypes.c_double
    lib.oracle_efq_rho.argtypes = []
    lib.oracle_efq_rho.restype = ctypes.c_double
    lib.oracle_efq_exponent.argtypes = [ctypes.c_double]
    lib.oracle_efq_exponent.restype = ci
    lib.oracle_efq_code.argtypes = [ctypes.c_double]
    lib.oracle_efq_code.restype = ci
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x):
    """Return (contiguous array, dtype code).  bf16 data is passed as its raw
    uint16 bit pattern; fp32 as float32."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle inputs are float32 arrays or bf16 bit patterns (uint16)")


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return _load().oracle_threads()


def scale_exponent(amax: float, rule: int) -> int:
    """Scale exponent e of a block whose largest magnitude is ``amax``."""
    return _load().oracle_scale_exponent(float(amax), int(rule))


def efq_beta() -> float:
    """Offset of the EFQ affine code rule (least-squares fit, see mxoracle.c)."""
    return _load().oracle_efq_beta()


def efq_rho() -> float:
    """Largest residual the EFQ block maximum may take."""
    return _load().oracle_efq_rho()


def efq_exponent(zmax: float) -> int:
    """EFQ block exponent from the block's largest log2 probability."""
    return _load().oracle_efq_exponent(float(zmax))


def efq_code(r: float) -> int:
    """EFQ code (0..7) of a log2 residual r = z - e_b."""
    return _load().oracle_efq_code(float(r))


def round_e2m1(v: float) -> int:
    """3-bit E2M1 magnitude code of a non-negative scaled value."""
    return _load().oracle_round_e2m1(float(v))


def quantize(x, rule: int):
    """Blocks of 32 along the flattened contiguous axis.

    Returns (codes uint8[n/2], scales uint8[n/32])."""
    x, dt = _as_input(x)
    n = x.size
    codes = np.empty(n // 2, np.uint8)
    scales = np.empty(n // BLOCK, np.uint8)
    rc = _load().oracle_quantize(_ptr(x), dt, n, int(rule), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle_quantize: n must be a multiple of 32")
    return codes, scales


def quantize_t(x, rule: int):
    """Blocks of 32 along the rows of a [rows, cols] matrix, output
    transposed: (codes [cols, rows_pad/2], scales [cols, rows_pad/32])."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    rp = (rows + BLOCK - 1) // BLOCK * BLOCK
    codes = np.empty((cols, rp // 2), np.uint8)
    scales = np.empty((cols, rp // BLOCK), np.uint8)
    rc = _load().oracle_quantize_t(_ptr(x), dt, rows, cols, int(rule), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle_quantize_t: bad shape")
    return codes, scales


def dequantize(codes, scales):
    """Binary64 values of packed codes under their E8M0 bytes."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    n = codes.size * 2
    y = np.empty(n, np.float64)
    rc = _load().oracle_dequantize(_ptr(codes), _ptr(scales), n, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_dequantize: bad sizes")
    return y


def attn_rows(q, k, v, *, causal: bool, mode: int, bc: int, rows,
              want_p: bool = False, want_tiles: bool = False, split: int = 0):
    """Attention output rows, binary64.

    q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] (float32 or bf16 bits as uint16).
    ``rows``: flattened (b*Hq + h)*Sq + i indices.  ``bc``: keys per KV
    tile (the running-max schedule).  ``split``: keys per split (a multiple
    of ``bc``; 0 = none): each split runs its own running max and the
    splits are merged in order.  Causal queries are aligned to the end of
    the keys (query i sees keys j <= i + Skv - Sq).  Returns a dict with
    ``o`` [n, D], ``l`` [n], ``m`` [n] and, on request,
    ``p_codes``/``p_scales`` and ``m_tiles``."""
    q, dt = _as_input(q)
    k, dt2 = _as_input(k)
    v, dt3 = _as_input(v)
    if not (dt == dt2 == dt3):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch")
    rows = np.ascontiguousarray(rows, np.int64)
    n = rows.size
    o = np.empty((n, D), np.float64)
    l_out = np.empty(n, np.float64)
    m_out = np.empty(n, np.float64)
    skv_pad = (Skv + BLOCK - 1) // BLOCK * BLOCK
    ntiles = (Skv + bc - 1) // bc
    pc = np.empty((n, skv_pad // 2), np.uint8) if want_p else None
    ps = np.empty((n, skv_pad // BLOCK), np.uint8) if want_p else None
    mt = np.empty((n, ntiles), np.float64) if want_tiles else None
    rc = _load().oracle_attn_rows_split(
        _ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
        int(mode), int(bc), int(split), _ptr(rows), n, _ptr(o), _ptr(l_out), _ptr(m_out),
        _ptr(mt), _ptr(pc), _ptr(ps))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows failed ({rc})")
    res = {"o": o, "l": l_out, "m": m_out}
    if want_p:
        res["p_codes"], res["p_scales"] = pc, ps
    if want_tiles:
        res["m_tiles"] = mt
    return res


def unpack_codes(codes):
    """Split packed bytes into 4-bit codes (element 2j = low nibble)."""
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def gemm_q(a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, rows=None,
           n_chunk: int = 2048):
    """W4A4 product of MXFP4 operands in binary64.

    The operands are stored as ``mxq_quantize`` writes row-major tensors:
    ``a`` [M, K] and ``b`` [N, K] with blocks of 32 along K (codes [rows,
    K/2], E8M0 bytes [rows, K/32]).  Returns ``(y, yabs)`` with
    y[m, n] = sum_k deq(a)[m, k] deq(b)[n, k] and yabs the same sum of
    absolute products (the scale of any rounding bound).  ``rows`` picks a
    subset of m (all when None).  A library matmul serves as the sum; the
    decode is ``dequantize``."""
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    a_codes = np.asarray(a_codes, np.uint8).reshape(M, K // 2)
    a_scales = np.asarray(a_scales, np.uint8).reshape(M, K // BLOCK)
    b_codes = np.asarray(b_codes, np.uint8).reshape(N, K // 2)
    b_scales = np.asarray(b_scales, np.uint8).reshape(N, K // BLOCK)
    rows = np.arange(M) if rows is None else np.asarray(rows, np.int64)
    A = dequantize(a_codes[rows], a_scales[rows]).reshape(rows.size, K)
    Aabs = np.abs(A)
    y = np.empty((rows.size, N), np.float64)
    yabs = np.empty((rows.size, N), np.float64)
    for n0 in range(0, N, n_chunk):
        n1 = min(N, n0 + n_chunk)
        Bt = dequantize(b_codes[n0:n1], b_scales[n0:n1]).reshape(n1 - n0, K).T
        y[:, n0:n1] = A @ Bt
        yabs[:, n0:n1] = Aabs @ np.abs(Bt)
    return y, yabs


def gemm(a, b, rule: int, rows=None):
    """Quantize ``a`` [M, K] and ``b`` [N, K] along K with ``rule``, then
    ``gemm_q``.  Returns (y, yabs, (a_codes, a_scales), (b_codes, b_scales))."""
    a, _ = _as_input(a)
    b, _ = _as_input(b)
    M, K = a.shape
    N, Kb = b.shape
    if Kb != K:
        raise ValueError("K mismatch")
    qa = quantize(a, rule)
    qb = quantize(b, rule)
    y, yabs = gemm_q(qa[0], qa[1], qb[0], qb[1], M, N, K, rows=rows)
    return y, yabs, qa, qb
