"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, and rejects bad arguments before any HIP
call."""
import ctypes
import os
import re

import pytest

import mxfp4_block_quantized_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx[a-z_0-9]*)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(mx.EXPORTS)


def test_library_exports_every_symbol():
    L = mx.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror():
    L = mx.lib()
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert len(L.mx_strerror(s)) > 3


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def test_quantize_rejects_bad_args():
    L = mx.lib()
    assert L.mxq_quantize(FAKE, 33, 1, 1, FAKE, FAKE, None) == -1      # n % 32
    assert L.mxq_quantize(FAKE, -32, 1, 1, FAKE, FAKE, None) == -1
    assert L.mxq_quantize(FAKE, 64, 5, 1, FAKE, FAKE, None) == -1      # dtype
    assert L.mxq_quantize(FAKE, 64, 1, 9, FAKE, FAKE, None) == -1      # mode
    assert L.mxq_quantize(None, 64, 1, 1, FAKE, FAKE, None) == -1      # null
    assert L.mxq_quantize(ctypes.c_void_p((1 << 20) + 4), 64, 1, 1, FAKE, FAKE, None) == -5
    assert L.mxq_quantize(None, 0, 1, 1, None, None, None) == 0        # empty is a no-op
    assert L.mxq_quantize_t(FAKE, 1, 64, 8, 1, 1, 48, FAKE, FAKE, None) == -1  # rows_pad % 32
    assert L.mxq_quantize_t(FAKE, 1, 64, 8, 1, 1, 32, FAKE, FAKE, None) == -1  # rows_pad < rows
    assert L.mxq_dequantize(FAKE, FAKE, 31, 0, FAKE, None) == -1
    assert L.mxq_dequantize(FAKE, FAKE, 64, 3, FAKE, None) == -1
    # past one dispatch's 2^32 work items (one thread per 16 / 8 elements)
    assert L.mxq_quantize(FAKE, 1 << 36, 1, 1, FAKE, FAKE, None) == -2
    assert L.mxq_dequantize(FAKE, FAKE, 1 << 35, 0, FAKE, None) == -2


def test_attention_rejects_bad_args():
    L = mx.lib()
    P = FAKE
    def fwd(dtype=1, B=1, Hq=2, Hkv=1, Sq=64, Skv=64, D=128, causal=0, mode=3, ws_bytes=1 << 40,
            q=P, ws=P):
        return L.mxattn_fwd(q, P, P, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, P, ws,
                            ctypes.c_size_t(ws_bytes), None)
    assert fwd(D=96) == -2
    assert fwd(Hq=3, Hkv=2) == -1
    assert fwd(causal=1, Skv=65) == -2
    assert fwd(mode=5) == -1
    assert fwd(dtype=2) == -1
    assert fwd(Sq=0) == -1
    assert fwd(q=None) == -1
    assert fwd(ws_bytes=16) == -3
    assert fwd(ws=None) == -3
    assert fwd(ws=ctypes.c_void_p((1 << 20) + 16)) == -5
    # the dump entry point needs the larger (Q~-holding) workspace
    nb = L.mxattn_workspace_bytes(1, 2, 1, 64, 64, 128, 1, 3)
    assert L.mxattn_fwd_dump(P, P, P, 1, 1, 2, 1, 64, 64, 128, 0, 3, P, P,
                             ctypes.c_size_t(nb), P, P, P, None) == -3
    # dump entry: FP16 mode has no P~ to dump
    assert L.mxattn_fwd_dump(P, P, P, 1, 1, 1, 1, 64, 64, 128, 0, 0, P, P,
                             ctypes.c_size_t(1 << 40), P, P, P, None) == -1


def test_workspace_and_tile_queries():
    L = mx.lib()
    assert L.mxattn_kv_tile(128, 3) == 128 and L.mxattn_kv_tile(64, 0) == 64
    assert L.mxattn_kv_tile(96, 3) == -2
    assert L.mxattn_workspace_bytes(1, 2, 1, 64, 64, 96, 1, 3) == 0
    nb = L.mxattn_workspace_bytes(1, 40, 40, 32760, 32760, 128, 1, 3)
    # K~ + V~^T tile images: 17408 bytes per 128 keys (0.53125 B per element
    # each), then one 4-byte arrival counter per (b, KV head) rounded to 256
    # bytes and the prefill work queue (8 words, 256 bytes); the Q~ regions
    # only in the dump size
    assert nb == 40 * 256 * 17408 + 256 + 256
    nd = L.mxattn_dump_workspace_bytes(1, 40, 40, 32760, 32760, 128, 1, 3)
    assert nd >= nb + 40 * 32760 * 128 * 17 // 32
    off, ld = mx.workspace_layout(1, 40, 40, 32760, 32760, 128, "bf16", "uos_pnq")
    assert ld == 32768 and off[2] == 0 and nb <= off[0] < off[1] and off[3:] == [17408, 0, 0]
    assert all(o % 256 == 0 for o in off[:3])
    assert off[1] + 40 * 32760 * 4 <= nd
    assert L.mxattn_dump_workspace_bytes(1, 40, 40, 32760, 32760, 128, 1, 0) == 0  # FP16
    off64, _ = mx.workspace_layout(1, 2, 2, 100, 100, 64, "f32", "ocp")
    assert off64[3] == 9216  # 8704 bytes for D = 64, rounded up to 1 KiB
    with pytest.raises(mx.MxError):
        mx.workspace_layout(1, 2, 2, 64, 64, 128, "bf16", "fp16")
    # K/V element count past 2^40 (its image size would overflow): rejected
    # even when Q is small (Sq = 1)
    assert L.mxattn_workspace_bytes(65535, 65535, 65535, 1, 1 << 20, 128, 1, 3) == 0
    assert L.mxattn_workspace_bytes(1, 8, 8, 1, (1 << 31) - 1, 128, 1, 3) == 0
    # launches whose work-item count would pass 2^32 in one grid dimension:
    # query tiles (65535 x 65535 heads, one tile each), K images (2^35
    # elements), fp32 Q of the FP16 mode (2^32 elements)
    assert L.mxattn_workspace_bytes(65535, 65535, 1, 1, 128, 64, 1, 3) == 0
    assert L.mxattn_workspace_bytes(1, 1, 1, 1, 1 << 28, 128, 1, 3) == 0
    assert L.mxattn_workspace_bytes(1, 1, 1, 1, (1 << 28) - 128, 128, 1, 3) > 0
    # past 2^31 K-image work items per (b, KV head): the image launches
    # count them in 64 bits (accepted shapes, D = 128 and 64)
    assert L.mxattn_workspace_bytes(1, 1, 1, 1, (1 << 27) + 128, 128, 1, 3) > 0
    assert L.mxattn_workspace_bytes(1, 1, 1, 1, (1 << 28) + 128, 64, 1, 3) > 0
    assert L.mxattn_workspace_bytes(1, 1, 1, 1 << 25, 128, 128, 0, 0) == 0
    assert L.mxattn_workspace_bytes(1, 1, 1, 1 << 25, 128, 128, 1, 0) > 0


def test_gemm_rejects_bad_args():
    L = mx.lib()
    P = FAKE
    big = 1 << 40
    def g(M=64, N=64, K=256, dt=0, a=P, sa=P, y=P, ws=P, wsb=big):
        return L.mxgemm(a, sa, P, P, M, N, K, dt, y, ws, wsb, None)
    assert g(K=96) == -2           # K % 128
    assert g(K=0) == -1
    assert g(M=0) == -1
    assert g(N=-3) == -1
    assert g(dt=4) == -1           # out dtype
    assert g(a=None) == -1
    assert g(y=None) == -1
    assert g(M=1 << 31) == -2
    # the per-lane 32-bit load offsets (row in tile x K/2) bound K
    kmax = ((((1 << 32) - 129) // 255) * 2) // 128 * 128
    assert 255 * (kmax // 2) + 128 < (1 << 32) <= 255 * ((kmax + 128) // 2) + 128
    assert L.mxgemm_workspace_bytes(64, 64, kmax) > 0
    assert L.mxgemm_workspace_bytes(64, 64, kmax + 128) == 0
    assert g(K=kmax + 128) == -2
    assert g(y=ctypes.c_void_p((1 << 20) + 8)) == -5   # y not 16-byte aligned
    assert g(ws=None) == -3
    assert g(wsb=16) == -3
    assert g(ws=ctypes.c_void_p((1 << 20) + 128)) == -5
    assert L.mxgemm_workspace_bytes(64, 64, 96) == 0
    # two scale images: ceil(rows/16) row tiles x ceil(K/512) groups x 256 B
    assert L.mxgemm_workspace_bytes(300, 20, 1024) == 19 * 2 * 256 + 2 * 2 * 256


def test_decode_rejects_bad_args():
    L = mx.lib()
    P = FAKE
    big = 1 << 40
    def d(dtype=1, B=1, Hq=8, Hkv=2, Sq=1, Skv=1000, D=128, causal=0, mode=3, ws=P, wsb=big, q=P):
        return L.mxattn_decode(q, P, P, dtype, B, Hq, Hkv, Sq, Skv, D, causal, mode, P, ws, wsb, None)
    assert d(mode=0) == -2                 # FP16 mode: use mxattn_fwd
    assert d(Sq=9) == -2                   # (Hq/Hkv) * Sq > 32
    assert d(D=96) == -2
    assert d(causal=1, Sq=4, Skv=3) == -2  # causal needs Sq <= Skv
    assert d(Hq=6, Hkv=4) == -1
    assert d(mode=5) == -1
    assert d(q=None) == -1
    assert d(ws=None) == -3
    assert d(wsb=10) == -3
    assert L.mxattn_decode_split(1, 8, 32768) % 128 == 0
    assert L.mxattn_decode_split(0, 8, 32768) == -1
    assert L.mxattn_decode_workspace_bytes(1, 8, 2, 1, 1000, 128, 1, 0) == 0
    assert L.mxattn_decode_workspace_bytes(1, 8, 2, 1, 1000, 128, 1, 3) > 0


def test_decode_split_and_workspace_sizes():
    """Split size: whole 128-key tiles, at least 4, about 1024 waves over
    all (b, KV head) groups, at most 1024 splits per group, never more than
    the keys.  Workspace: the prepare layout (KV images, one arrival counter
    per (b, KV head) rounded to 256 bytes, the Q~ regions) followed by the
    partial states, 32 query columns of D + 4 floats per split; the prefill
    work queue (8 words) after the counters."""
    L = mx.lib()
    assert L.mxattn_decode_split(8, 8, 32768) == 16 * 128    # 64 groups x 16 splits
    assert L.mxattn_decode_split(1, 8, 32768) == 4 * 128     # the 4-tile floor
    assert L.mxattn_decode_split(1, 1, 1 << 20) == 8 * 128   # 1024 splits
    assert L.mxattn_decode_split(1, 1, 300) == 3 * 128       # all the keys
    for B, Hq, Hkv, Sq, Skv, D in ((8, 32, 8, 1, 32768, 128), (3, 8, 2, 2, 5000, 64)):
        split = L.mxattn_decode_split(B, Hkv, Skv)
        nsplit = -(-((Skv + 127) // 128 * 128) // split)
        dump = L.mxattn_dump_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, 1, 3)
        part = B * Hkv * nsplit * 32 * (D + 4) * 4
        got = L.mxattn_decode_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, 1, 3)
        assert got == (dump + 255) // 256 * 256 + part, (B, Skv, got, dump, part)
        nb = L.mxattn_workspace_bytes(B, Hq, Hkv, Sq, Skv, D, 1, 3)
        img = B * Hkv * ((Skv + 127) // 128) * (17408 if D == 128 else 9216)
        assert nb == img + (B * Hkv * 4 + 255) // 256 * 256 + 256


def test_varlen_rejects_bad_args():
    L = mx.lib()
    P = FAKE
    big = 1 << 40
    odd = ctypes.c_void_p((1 << 20) + 2)

    def f(mode=3, lq=P, lk=P, slot=None, pc=None, ps=None, causal=1, Sq=200, Skv=300, D=128):
        return L.mxattn_fwd_varlen(P, P, P, 1, 2, 4, 2, Sq, Skv, D, lq, lk, causal, mode, P, P,
                                   big, slot, pc, ps, None)

    def d(lk=P, slot=None, pc=None, ps=None, Sq=1, mode=3):
        return L.mxattn_decode_varlen(P, P, P, 1, 2, 8, 2, Sq, 4000, 128, lk, 1, mode, P, P, big,
                                      slot, pc, ps, None)

    assert f(mode=0) == -2          # FP16 mode has no varlen form
    assert f(D=80) == -2
    assert f(lq=None) == -1 and f(lk=None) == -1
    assert f(lk=odd) == -5
    assert f(slot=P) == -1          # dump pointers: all or none
    assert f(slot=P, pc=P) == -1
    assert f(causal=2) == -1
    assert d(lk=None) == -1
    assert d(lk=odd) == -5
    assert d(pc=P) == -1
    assert d(Sq=9) == -2            # (Hq/Hkv) * Sq > 32
    assert d(mode=0) == -2
    assert L.mxattn_prepare_varlen(P, P, P, 1, 2, 8, 2, 1, 4000, 128, None, 3, P, big, None) == -1
    assert L.mxattn_prepare_varlen(P, P, P, 1, 2, 8, 2, 1, 4000, 128, P, 0, P, big, None) == -2
    assert L.mxattn_decode_varlen_prepared(P, 1, 2, 8, 2, 1, 4000, 128, None, 1, 3, P, P, big,
                                           None) == -1
    assert L.mxattn_decode_varlen_prepared(P, 1, 2, 8, 2, 1, 4000, 128, odd, 1, 3, P, P, big,
                                           None) == -5
