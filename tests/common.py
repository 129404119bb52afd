"""Shared helpers for the GPU parity tests (inputs come from mxsynth; the
expected values from the oracle)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import mxsynth  # noqa: E402
import oracle  # noqa: E402

MODE_IDS = {"fp16": oracle.MODE_FP16, "ocp": oracle.MODE_OCP, "uos": oracle.MODE_UOS,
            "uos_pnq": oracle.MODE_UOS_PNQ, "uos_efq": oracle.MODE_UOS_EFQ}
RULE_IDS = {"ocp": oracle.RULE_OCP, "uos": oracle.RULE_UOS}
RULE_OF_MODE = {"ocp": "ocp", "uos": "uos", "uos_pnq": "uos", "uos_efq": "uos"}

# Output tolerance of the attention parity tests (O is O(1)).
MAX_ABS = 2e-3
MEAN_ABS = 2e-4
# Largest admissible fraction of P~ elements whose value differs from the
# oracle's (fp32 exp / fp32 accumulation versus binary64 near a rounding
# boundary of the E2M1 grid).
FLIP_MAX = 1e-4


def gpu():
    """The torch module, skipping the test when no GPU or no library."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_block_quantized_amd as mx
    mx.lib()  # raises if the HIP library is missing: no silent fallback
    return torch, mx


def to_torch(a, device="cuda"):
    """numpy float32 / bf16 bits (uint16) -> torch tensor on the GPU."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def np_u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def flips(gpu_codes, gpu_scales, ref_codes, ref_scales, nkeys):
    """Fraction of P~ elements (over the first nkeys keys of each row) whose
    dequantized value differs, and the fraction of differing scale bytes."""
    nb = (nkeys + 31) // 32
    gc = oracle.unpack_codes(gpu_codes[:, : nb * 16])[:, :nkeys]
    rc = oracle.unpack_codes(ref_codes[:, : nb * 16])[:, :nkeys]
    gs = np.repeat(gpu_scales[:, :nb].astype(np.int64), 32, axis=1)[:, :nkeys]
    rs = np.repeat(ref_scales[:, :nb].astype(np.int64), 32, axis=1)[:, :nkeys]
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    gv = mag[gc & 7] * np.exp2(gs - 127.0)
    rv = mag[rc & 7] * np.exp2(rs - 127.0)
    diff = gv != rv
    sdiff = gpu_scales[:, :nb] != ref_scales[:, :nb]
    return float(diff.mean()), float(sdiff.mean()), int(diff.sum())


def decode_kv_images(w, off, B, Hkv, Skv, D):
    """Read the KV tile images of a workspace (layout documented in
    include/mxattn.h) back into plain arrays: K~ codes [B*Hkv][rows][D/2],
    K~ scales [B*Hkv][rows][D/32], V~^T codes [B*Hkv][D][rows/2], V~^T
    scales [B*Hkv][D][rows/32] with rows = Skv rounded up to 128, plus the
    padding bytes at the end of each image, which must be zero."""
    BG, IMG = B * Hkv, off[3]
    nt = (Skv + 127) // 128
    DH, NC = D // 64, D // 32
    im = w[off[2]:off[2] + BG * nt * IMG].reshape(BG, nt, IMG)
    # K~: [subtile t][d-half i][lane l][16]; lane l of (t, i) holds the key
    # 64 (t/2) + 32 (R/4 % 2) + 16 (t%2) + 4 (R/8) + R%4 (R = l%32) of the
    # tile, elements 32 (2 i + l/32) .. +31
    T, t, i, l = np.meshgrid(np.arange(nt), np.arange(4), np.arange(DH), np.arange(64), indexing="ij")
    R = l % 32
    krow = T * 128 + 64 * (t // 2) + 32 * ((R // 4) % 2) + 16 * (t % 2) + 4 * (R // 8) + R % 4
    kblk = 2 * i + l // 32
    kc = im[:, :, :64 * D].reshape(BG, nt, 4, DH, 64, 16)
    ksc = im[:, :, 128 * D:132 * D].reshape(BG, nt, 64, D // 16)
    k_codes = np.zeros((BG, nt * 128, D // 32, 16), np.uint8)
    k_scales = np.zeros((BG, nt * 128, D // 32), np.uint8)
    k_codes[:, krow, kblk, :] = kc[:, T, t, i, l, :]
    k_scales[:, krow, kblk] = ksc[:, T, l, t * DH + i]
    # V~^T: [channel tile c][key step s][lane l][16]; lane l holds channel
    # 32 c + l%32, keys 64 s + 32 (l/32) .. +31 of the tile
    T, c, s_, l = np.meshgrid(np.arange(nt), np.arange(NC), np.arange(2), np.arange(64), indexing="ij")
    ch = 32 * c + l % 32
    vblk = T * 4 + 2 * s_ + l // 32
    vc = im[:, :, 64 * D:128 * D].reshape(BG, nt, NC, 2, 64, 16)
    vsc = im[:, :, 132 * D:136 * D].reshape(BG, nt, 64, D // 16)
    vt_codes = np.zeros((BG, D, nt * 4, 16), np.uint8)
    vt_scales = np.zeros((BG, D, nt * 4), np.uint8)
    vt_codes[:, ch, vblk, :] = vc[:, T, c, s_, l, :]
    vt_scales[:, ch, vblk] = vsc[:, T, l, 2 * c + s_]
    pad = im[:, :, 136 * D:]
    return (k_codes.reshape(BG, nt * 128, D // 2), k_scales,
            vt_codes.reshape(BG, D, nt * 64), vt_scales, pad)
