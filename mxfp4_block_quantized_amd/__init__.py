"""Python binding of ``libmxattn.so``: MXFP4 block quantization and MXFP4
attention (OCP, UOS, UOS+PNQ and the unquantized FP16 mode) on gfx950.

This module only marshals arguments: it takes PyTorch device tensors (used
for memory and streams), passes their pointers to the C ABI declared in
``include/mxattn.h`` and raises on any non-zero status.  Every step of the
computation runs in the HIP kernels of ``csrc/``.  There is no CPU path: if
the library is missing this module raises at first use.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxattn.so")

MX_F32, MX_BF16 = 0, 1
MXQ_OCP, MXQ_UOS = 0, 1
MXATTN_FP16, MXATTN_OCP, MXATTN_UOS, MXATTN_UOS_PNQ, MXATTN_UOS_EFQ = 0, 1, 2, 3, 4
MODES = {"fp16": MXATTN_FP16, "ocp": MXATTN_OCP, "uos": MXATTN_UOS, "uos_pnq": MXATTN_UOS_PNQ,
         "uos_efq": MXATTN_UOS_EFQ}
RULES = {"ocp": MXQ_OCP, "uos": MXQ_UOS}

# Symbols the header declares; the CPU tests check the library exports them.
EXPORTS = (
    "mx_strerror", "mxq_quantize", "mxq_quantize_t", "mxq_dequantize",
    "mxattn_workspace_bytes", "mxattn_dump_workspace_bytes", "mxattn_workspace_layout",
    "mxattn_kv_tile",
    "mxattn_fwd", "mxattn_fwd_dump", "mxattn_prepare", "mxattn_fwd_prepared", "mxgemm",
    "mxgemm_workspace_bytes", "mxattn_decode_split", "mxattn_decode_workspace_bytes",
    "mxattn_decode", "mxattn_decode_prepared", "mxattn_decode_dump", "mxattn_fwd_varlen",
    "mxattn_decode_varlen", "mxattn_prepare_varlen", "mxattn_decode_varlen_prepared",
    "mxgemm_noalloc",
)

_lib = None


class MxError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({lib().mx_strerror(status).decode()})")
        self.status = status


def lib():
    """Load ``libmxattn.so`` (built by ``build.py``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mxfp4_block_quantized_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.mx_strerror.argtypes = [ci]
    L.mx_strerror.restype = ctypes.c_char_p
    L.mxq_quantize.argtypes = [P, i64, ci, ci, P, P, P]
    L.mxq_quantize_t.argtypes = [P, i64, i64, i64, ci, ci, i64, P, P, P]
    L.mxq_dequantize.argtypes = [P, P, i64, ci, P, P]
    L.mxattn_workspace_bytes.argtypes = [ci] * 8
    L.mxattn_workspace_bytes.restype = sz
    L.mxattn_dump_workspace_bytes.argtypes = [ci] * 8
    L.mxattn_dump_workspace_bytes.restype = sz
    L.mxattn_workspace_layout.argtypes = [ci] * 8 + [ctypes.POINTER(sz), ctypes.POINTER(i64)]
    L.mxattn_kv_tile.argtypes = [ci, ci]
    L.mxattn_fwd.argtypes = [P, P, P] + [ci] * 9 + [P, P, sz, P]
    L.mxattn_fwd_dump.argtypes = [P, P, P] + [ci] * 9 + [P, P, sz, P, P, P, P]
    L.mxattn_prepare.argtypes = [P, P, P] + [ci] * 8 + [P, sz, P]
    L.mxattn_fwd_prepared.argtypes = [P, P] + [ci] * 9 + [P, P, sz, P]
    L.mxgemm.argtypes = [P, P, P, P, i64, i64, i64, ci, P, P, sz, P]
    L.mxattn_decode_split.argtypes = [ci, ci, ci]
    L.mxattn_decode_workspace_bytes.argtypes = [ci] * 8
    L.mxattn_decode_workspace_bytes.restype = sz
    L.mxattn_decode.argtypes = [P, P, P] + [ci] * 9 + [P, P, sz, P]
    L.mxattn_decode_prepared.argtypes = [P] + [ci] * 9 + [P, P, sz, P]
    L.mxattn_decode_dump.argtypes = [P, P, P] + [ci] * 9 + [P, P, sz, P, P, P, P]
    L.mxattn_fwd_varlen.argtypes = [P, P, P] + [ci] * 7 + [P, P, ci, ci, P, P, sz, P, P, P, P]
    L.mxattn_decode_varlen.argtypes = [P, P, P] + [ci] * 7 + [P, ci, ci, P, P, sz, P, P, P, P]
    L.mxattn_prepare_varlen.argtypes = [P, P, P] + [ci] * 7 + [P, ci, P, sz, P]
    L.mxattn_decode_varlen_prepared.argtypes = [P] + [ci] * 7 + [P, ci, ci, P, P, sz, P]
    L.mxgemm_noalloc.argtypes = [P, P, P, P, i64, i64, i64, ci, P, P]
    L.mxgemm_workspace_bytes.argtypes = [i64, i64, i64]
    L.mxgemm_workspace_bytes.restype = sz
    for f in ("mxq_quantize", "mxq_quantize_t", "mxq_dequantize", "mxattn_workspace_layout",
              "mxattn_kv_tile", "mxattn_fwd", "mxattn_fwd_dump", "mxattn_prepare",
              "mxattn_fwd_prepared", "mxgemm", "mxattn_decode_split", "mxattn_decode",
              "mxattn_decode_prepared", "mxattn_decode_dump", "mxattn_fwd_varlen",
              "mxattn_decode_varlen", "mxattn_prepare_varlen", "mxattn_decode_varlen_prepared",
              "mxgemm_noalloc"):
        getattr(L, f).restype = ci
    _lib = L
    return L


def _check(fn, status):
    if status != 0:
        raise MxError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MX_F32
    if t.dtype == torch.bfloat16:
        return MX_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run ``fn`` with its ``stream`` argument as torch's current stream, so
    that every temporary it makes (workspace, length arrays, dump buffers,
    zero-filled outputs) is allocated, filled and released on the stream
    the kernels are launched on.  Without this, the caching allocator could
    hand a freed temporary to work on another stream while a kernel still
    reads it.  The caller orders its own inputs with that stream."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return wrapper


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _mode(mode, table):
    return table[mode] if isinstance(mode, str) else int(mode)


def _dev(t, name, dtype=None, numel=None):
    """``t`` must be a contiguous GPU tensor (of ``dtype``, with at least
    ``numel`` elements): the library reads and writes raw device memory."""
    if not torch.is_tensor(t) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs {numel} elements, has {t.numel()}")
    return t


def _attn_shapes(q, k, v=None, *, k_data=True):
    """(B, Hq, Hkv, Sq, Skv, D) of q [B,Hq,Sq,D] and k (and v) [B,Hkv,Skv,D],
    one dtype throughout; ``k_data=False``: k gives the key shape only."""
    _dev(q, "q")
    _dtype_code(q)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D: [B, heads, rows, D]")
    if k_data:
        _dev(k, "k", q.dtype)
    if v is not None:
        _dev(v, "v", q.dtype)
        if v.shape != k.shape:
            raise ValueError(f"v {tuple(v.shape)} differs from k {tuple(k.shape)}")
    B, Hq, Sq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} differ in batch or D")
    return B, Hq, k.shape[1], Sq, k.shape[2], D


def _out(out, shape, device, zero=False):
    """The fp32 output [B,Hq,Sq,D]: allocated, or the caller's, checked."""
    if out is None:
        return (torch.zeros if zero else torch.empty)(shape, dtype=torch.float32, device=device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out: expected shape {tuple(shape)}, got {tuple(out.shape)}")
    return out


def _ws(workspace):
    return _dev(workspace, "workspace", torch.uint8)


# ------------------------------------------------------------ quantizer ----

@_on_stream
def quantize(x: torch.Tensor, mode="uos", codes=None, scales=None, stream=None):
    """Blocks of 32 along the flattened contiguous axis of ``x`` (fp32 or
    bf16, numel % 32 == 0).  Returns (codes uint8[n/2], scales uint8[n/32])."""
    _dev(x, "x")
    n = x.numel()
    if codes is None:
        codes = torch.empty(n // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(n // 32, dtype=torch.uint8, device=x.device)
    _dev(codes, "codes", torch.uint8, n // 2)
    _dev(scales, "scales", torch.uint8, n // 32)
    _check("mxq_quantize", lib().mxq_quantize(_ptr(x), n, _dtype_code(x), _mode(mode, RULES),
                                              _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


@_on_stream
def quantize_t(x: torch.Tensor, mode="uos", rows_pad: int = 0, stream=None):
    """Blocks of 32 along the rows of ``x`` [batch, rows, cols] (or [rows,
    cols]); returns transposed (codes [batch, cols, rows_pad/2], scales
    [batch, cols, rows_pad/32])."""
    _dev(x, "x")
    if x.dim() not in (2, 3):
        raise ValueError("x must be [rows, cols] or [batch, rows, cols]")
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    batch, rows, cols = x3.shape
    rp = rows_pad or (rows + 31) // 32 * 32
    codes = torch.empty((batch, cols, rp // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((batch, cols, rp // 32), dtype=torch.uint8, device=x.device)
    _check("mxq_quantize_t", lib().mxq_quantize_t(
        _ptr(x3), batch, rows, cols, _dtype_code(x), _mode(mode, RULES), rp,
        _ptr(codes), _ptr(scales), _stream(stream)))
    if x.dim() == 2:
        return codes[0], scales[0]
    return codes, scales


@_on_stream
def dequantize(codes: torch.Tensor, scales: torch.Tensor, out_dtype=torch.float32,
               out=None, stream=None):
    """Values of packed codes under their E8M0 bytes, as fp32 or bf16."""
    _dev(codes, "codes", torch.uint8)
    n = codes.numel() * 2
    _dev(scales, "scales", torch.uint8, n // 32)
    if out is None:
        out = torch.empty(n, dtype=out_dtype, device=codes.device)
    _dev(out, "out", None, n)
    _check("mxq_dequantize", lib().mxq_dequantize(_ptr(codes), _ptr(scales), n,
                                                  _dtype_code(out), _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------ attention ----

def kv_tile(D: int, mode="uos_pnq") -> int:
    """Keys per KV tile: the running-max schedule the oracle must mirror."""
    r = lib().mxattn_kv_tile(D, _mode(mode, MODES))
    if r < 0:
        raise MxError("mxattn_kv_tile", r)
    return r


def workspace_bytes(B, Hq, Hkv, Sq, Skv, D, dtype, mode, dump=False) -> int:
    """Workspace of attn_fwd (``dump``: of the dump entry points, which also
    store the kernel's Q~)."""
    dt = MX_BF16 if dtype in (torch.bfloat16, "bf16", MX_BF16) else MX_F32
    f = lib().mxattn_dump_workspace_bytes if dump else lib().mxattn_workspace_bytes
    return f(B, Hq, Hkv, Sq, Skv, D, dt, _mode(mode, MODES))


def workspace_layout(B, Hq, Hkv, Sq, Skv, D, dtype, mode):
    """([Q~ codes offset, Q~ scales offset, KV tile images offset (0), bytes
    per image, 0, 0], skv_ld) — for reading the quantized operands back
    (image layout in include/mxattn.h; the Q~ regions exist in a dump-sized
    workspace)."""
    dt = MX_BF16 if dtype in (torch.bfloat16, "bf16", MX_BF16) else MX_F32
    off = (ctypes.c_size_t * 6)()
    ld = ctypes.c_int64()
    _check("mxattn_workspace_layout", lib().mxattn_workspace_layout(
        B, Hq, Hkv, Sq, Skv, D, dt, _mode(mode, MODES), off, ctypes.byref(ld)))
    return list(off), ld.value


def alloc_workspace(q, k, mode, dump=False):
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, k_data=False)
    nb = workspace_bytes(B, Hq, Hkv, Sq, Skv, D, q.dtype, mode, dump)
    if nb == 0:
        raise ValueError("invalid attention shape")
    # torch's caching allocator returns >= 512-byte aligned blocks
    return torch.empty(nb, dtype=torch.uint8, device=q.device)


@_on_stream
def attn_fwd(q, k, v, *, causal=False, mode="uos_pnq", out=None, workspace=None,
             stream=None):
    """O = softmax(q k^T / sqrt(D)) v in the given mode; fp32 output.
    q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D]; fp32 or bf16, contiguous, on the GPU."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    out = _out(out, (B, Hq, Sq, D), q.device)
    if workspace is None:
        workspace = alloc_workspace(q, k, mode)
    _ws(workspace)
    _check("mxattn_fwd", lib().mxattn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
        _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


@_on_stream
def attn_prepare(q, k, v, *, mode="uos_pnq", workspace=None, stream=None):
    """First half of attn_fwd: quantize (or convert) the key/value operands
    into the workspace (Q is quantized inside the attention kernels).
    Returns the workspace."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    if workspace is None:
        workspace = alloc_workspace(q, k, mode)
    _ws(workspace)
    _check("mxattn_prepare", lib().mxattn_prepare(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, _mode(mode, MODES),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


@_on_stream
def attn_fwd_prepared(q, k, workspace, *, causal=False, mode="uos_pnq", out=None,
                      stream=None):
    """Second half of attn_fwd: the fused attention kernel for the queries q
    on a workspace filled by attn_prepare with the same shapes, dtype and
    mode."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, k_data=False)
    out = _out(out, (B, Hq, Sq, D), q.device)
    _ws(workspace)
    _check("mxattn_fwd_prepared", lib().mxattn_fwd_prepared(
        _ptr(q), _ptr(k), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
        _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


@_on_stream
def attn_fwd_dump(q, k, v, rows, *, causal=False, mode="uos_pnq", workspace=None,
                  stream=None):
    """attn_fwd plus the P~ codes / E8M0 bytes of the flattened query rows
    ``rows`` ((b*Hq + h)*Sq + i).  Returns (o, p_codes [n, skv_ld/2],
    p_scales [n, skv_ld/32], workspace); unvisited key blocks stay zero.
    The workspace also holds the kernel's Q~ (workspace_layout off[0:2])."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    n, slot, pc, ps = _dump_buffers(q, rows, B, Hq, Sq, (Skv + 127) // 128 * 128)
    out = _out(None, (B, Hq, Sq, D), q.device)
    if workspace is None:
        workspace = alloc_workspace(q, k, mode, dump=True)
    _ws(workspace)
    _check("mxattn_fwd_dump", lib().mxattn_fwd_dump(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
        _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(), _ptr(slot),
        _ptr(pc), _ptr(ps), _stream(stream)))
    return out, pc[:n], ps[:n], workspace


# ------------------------------------------------- short-query (decode) ----

def decode_split(B: int, Hkv: int, Skv: int) -> int:
    """Keys per split of attn_decode for this shape: the schedule the
    oracle must mirror (attn_rows(..., split=...))."""
    r = lib().mxattn_decode_split(B, Hkv, Skv)
    if r < 0:
        raise MxError("mxattn_decode_split", r)
    return r


def alloc_decode_workspace(q, k, mode):
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, k_data=False)
    dt = _dtype_code(q)
    nb = lib().mxattn_decode_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, dt, _mode(mode, MODES))
    if nb == 0:
        raise ValueError("invalid or unsupported decode shape")
    return torch.empty(nb, dtype=torch.uint8, device=q.device)


@_on_stream
def attn_decode(q, k, v, *, causal=False, mode="uos_pnq", out=None, workspace=None,
                stream=None):
    """Short-query attention over key splits (fp32 output); causal queries
    are aligned to the end of the keys.  q [B,Hq,Sq,D] with (Hq/Hkv)*Sq <=
    32, k/v [B,Hkv,Skv,D]."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    out = _out(out, (B, Hq, Sq, D), q.device)
    if workspace is None:
        workspace = alloc_decode_workspace(q, k, mode)
    _ws(workspace)
    _check("mxattn_decode", lib().mxattn_decode(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
        _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


@_on_stream
def attn_decode_prepared(q, k, workspace, *, causal=False, mode="uos_pnq", out=None,
                         stream=None):
    """attn_decode of the queries q on a workspace filled by attn_prepare
    (the key shape from k, whose data is not read)."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, k_data=False)
    out = _out(out, (B, Hq, Sq, D), q.device)
    _ws(workspace)
    _check("mxattn_decode_prepared", lib().mxattn_decode_prepared(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)), _mode(mode, MODES),
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


@_on_stream
def attn_decode_dump(q, k, v, rows, *, causal=False, mode="uos_pnq", workspace=None,
                     stream=None):
    """attn_decode plus the P~ codes / E8M0 bytes of the flattened query
    rows ``rows``; returns (o, p_codes, p_scales, workspace), the workspace
    holding the kernel's Q~ as for attn_fwd_dump."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    n, slot, pc, ps = _dump_buffers(q, rows, B, Hq, Sq, (Skv + 127) // 128 * 128)
    out = _out(None, (B, Hq, Sq, D), q.device)
    if workspace is None:
        workspace = alloc_decode_workspace(q, k, mode)
    _ws(workspace)
    _check("mxattn_decode_dump", lib().mxattn_decode_dump(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
        _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(), _ptr(slot),
        _ptr(pc), _ptr(ps), _stream(stream)))
    return out, pc[:n], ps[:n], workspace


# ------------------------------------------------------------ W4A4 GEMM ----

def gemm_workspace(M: int, N: int, K: int, device="cuda"):
    """Workspace for ``gemm`` at this shape (uint8 device tensor)."""
    n = lib().mxgemm_workspace_bytes(M, N, K)
    if n == 0:
        raise MxError("mxgemm_workspace_bytes", -1)
    return torch.empty(n, dtype=torch.uint8, device=device)


@_on_stream
def gemm(a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int,
         out_dtype=torch.float32, out=None, workspace=None, stream=None):
    """y [M, N] = deq(a) deq(b)^T for MXFP4 operands stored as ``quantize``
    writes row-major a [M, K] and b [N, K] (K % 128 == 0)."""
    _dev(a_codes, "a_codes", torch.uint8, M * K // 2)
    _dev(a_scales, "a_scales", torch.uint8, M * K // 32)
    _dev(b_codes, "b_codes", torch.uint8, N * K // 2)
    _dev(b_scales, "b_scales", torch.uint8, N * K // 32)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _dev(out, "out", None, M * N)
    if workspace is None:
        workspace = gemm_workspace(M, N, K, a_codes.device)
    _ws(workspace)
    _check("mxgemm", lib().mxgemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                                  M, N, K, _dtype_code(out), _ptr(out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))
    return out


@_on_stream
@_on_stream
def gemm_noalloc(a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, out,
                 stream=None):
    """``gemm`` into the caller's ``out`` [M, N] (fp32 or bf16) with the
    library's own scratch instead of a workspace: the C call allocates
    nothing.  Calls that overlap on one GPU race (one shared scratch)."""
    _dev(a_codes, "a_codes", torch.uint8, M * K // 2)
    _dev(a_scales, "a_scales", torch.uint8, M * K // 32)
    _dev(b_codes, "b_codes", torch.uint8, N * K // 2)
    _dev(b_scales, "b_scales", torch.uint8, N * K // 32)
    _dev(out, "out", None, M * N)
    _check("mxgemm_noalloc", lib().mxgemm_noalloc(
        _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K, _dtype_code(out),
        _ptr(out), _stream(stream)))
    return out


def linear_w4a4(x: torch.Tensor, w_codes, w_scales, N: int, mode="uos",
                out_dtype=torch.bfloat16, out=None, workspace=None, stream=None):
    """x [M, K] (fp32 or bf16) quantized along K with ``mode``, times the
    MXFP4 weight (w_codes [N, K/2], w_scales [N, K/32]): y [M, N]."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    xc, xs = quantize(x.contiguous(), mode, stream=stream)
    return gemm(xc, xs, w_codes, w_scales, M, N, K, out_dtype=out_dtype, out=out,
                workspace=workspace, stream=stream)


# ------------------------------------------------ per-sequence lengths ----

def _dump_buffers(q, rows, B, Hq, Sq, skv_ld):
    """Slot table and P~ buffers of the flattened query rows ``rows``."""
    rows = torch.as_tensor(rows, dtype=torch.int64).reshape(-1)
    n = rows.numel()
    if n and (int(rows.min()) < 0 or int(rows.max()) >= B * Hq * Sq):
        raise ValueError("rows: flattened query rows must lie in [0, B*Hq*Sq)")
    slot = torch.full((B * Hq * Sq,), -1, dtype=torch.int32)
    slot[rows] = torch.arange(n, dtype=torch.int32)
    slot = slot.to(q.device)
    pc = torch.zeros((max(n, 1), skv_ld // 2), dtype=torch.uint8, device=q.device)
    ps = torch.zeros((max(n, 1), skv_ld // 32), dtype=torch.uint8, device=q.device)
    return n, slot, pc, ps


def _lens(x, B, device):
    """Per-entry lengths as a device int32 array of B entries (a GPU int32
    tensor of that size is used as is)."""
    if torch.is_tensor(x) and x.is_cuda and x.dtype == torch.int32 and x.is_contiguous():
        t = x
    else:
        t = torch.as_tensor(x).to(dtype=torch.int32, device=device).contiguous()
    if t.numel() != B:
        raise ValueError(f"lengths: expected {B} entries, got {t.numel()}")
    return t


@_on_stream
def attn_fwd_varlen(q, k, v, seqlens_q, seqlens_k, *, causal=False, mode="uos_pnq", out=None,
                    workspace=None, rows=None, stream=None):
    """Padded batch of sequences with their own lengths: entry b has
    seqlens_q[b] query rows and seqlens_k[b] keys (q [B,Hq,Sq,D], k/v
    [B,Hkv,Skv,D] padded).  Rows past an entry's length are not written
    (``out`` defaults to zeros).  With ``rows`` (flattened query rows), also
    returns the P~ dump: (o, p_codes, p_scales, workspace)."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    lq, lk = _lens(seqlens_q, B, q.device), _lens(seqlens_k, B, q.device)
    out = _out(out, (B, Hq, Sq, D), q.device, zero=True)
    if workspace is None:
        workspace = alloc_workspace(q, k, mode, dump=rows is not None)
    _ws(workspace)
    slot = pc = ps = None
    if rows is not None:
        n, slot, pc, ps = _dump_buffers(q, rows, B, Hq, Sq, (Skv + 127) // 128 * 128)
    _check("mxattn_fwd_varlen", lib().mxattn_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, _ptr(lq), _ptr(lk),
        int(bool(causal)), _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(),
        _ptr(slot), _ptr(pc), _ptr(ps), _stream(stream)))
    if rows is None:
        return out
    return out, pc[:n], ps[:n], workspace


@_on_stream
def attn_decode_varlen(q, k, v, seqlens_k, *, causal=False, mode="uos_pnq", out=None,
                       workspace=None, rows=None, stream=None):
    """Short-query attention over key splits for a padded KV cache whose
    entry b holds seqlens_k[b] keys (q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D]).
    Rows that see no key are not written (``out`` defaults to zeros).  With
    ``rows``, also returns the P~ dump: (o, p_codes, p_scales, workspace)."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    lk = _lens(seqlens_k, B, q.device)
    out = _out(out, (B, Hq, Sq, D), q.device, zero=True)
    if workspace is None:
        workspace = alloc_decode_workspace(q, k, mode)
    _ws(workspace)
    slot = pc = ps = None
    if rows is not None:
        n, slot, pc, ps = _dump_buffers(q, rows, B, Hq, Sq, (Skv + 127) // 128 * 128)
    _check("mxattn_decode_varlen", lib().mxattn_decode_varlen(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, _ptr(lk),
        int(bool(causal)), _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(),
        _ptr(slot), _ptr(pc), _ptr(ps), _stream(stream)))
    if rows is None:
        return out
    return out, pc[:n], ps[:n], workspace


@_on_stream
def attn_prepare_varlen(q, k, v, seqlens_k, *, mode="uos_pnq", workspace=None, stream=None):
    """KV tile images of a padded KV cache whose entry b holds seqlens_k[b]
    keys (keys past it quantized as zero), for attn_decode_varlen_prepared.
    Returns the workspace (decode-sized unless one is given)."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, v)
    lk = _lens(seqlens_k, B, q.device)
    if workspace is None:
        workspace = alloc_decode_workspace(q, k, mode)
    _ws(workspace)
    _check("mxattn_prepare_varlen", lib().mxattn_prepare_varlen(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, _ptr(lk),
        _mode(mode, MODES), _ptr(workspace), workspace.numel(), _stream(stream)))
    return workspace


@_on_stream
def attn_decode_varlen_prepared(q, k, workspace, seqlens_k, *, causal=False, mode="uos_pnq",
                                out=None, stream=None):
    """attn_decode_varlen on a workspace filled by attn_prepare_varlen with
    the same lengths (the key shape from k, whose data is not read)."""
    B, Hq, Hkv, Sq, Skv, D = _attn_shapes(q, k, k_data=False)
    lk = _lens(seqlens_k, B, q.device)
    out = _out(out, (B, Hq, Sq, D), q.device, zero=True)
    _ws(workspace)
    _check("mxattn_decode_varlen_prepared", lib().mxattn_decode_varlen_prepared(
        _ptr(q), _dtype_code(q), B, Hq, Hkv, Sq, Skv, D, _ptr(lk), int(bool(causal)),
        _mode(mode, MODES), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out
