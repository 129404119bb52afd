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
            "uos_pnq": oracle.MODE_UOS_PNQ}
RULE_IDS = {"ocp": oracle.RULE_OCP, "uos": oracle.RULE_UOS}
RULE_OF_MODE = {"ocp": "ocp", "uos": "uos", "uos_pnq": "uos"}

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
