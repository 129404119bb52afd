"""Build the HIP library ``libmxattn.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmxattn.so")

SOURCES = ["capi.cpp", "quant.hip", "attn_mx.hip", "attn_f16.hip", "gemm_mx.hip"]
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of every device code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


# Extra flags per source.  The attention kernels handle no NaNs (inputs
# are finite; masking uses -inf), so max/min need no NaN-quieting
# canonicalisation of the matrix-core results.
EXTRA_FLAGS = {
    # both attention kernels interleave matrix and vector work in fenced
    # regions that follow the source order: instruction selection keeps that
    # order, and machine sinking would move matrix instructions across the
    # uniform branches between the regions
    "attn_mx.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-pre-RA-sched=source",
                    "-mllvm", "-disable-machine-sink"],
    "attn_f16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-pre-RA-sched=source",
                     "-mllvm", "-disable-machine-sink"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns about the device-only target feature; drop that
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libmxattn.so`` (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        flags = [f for f in HIPCC_FLAGS if f != "-shared"] + EXTRA_FLAGS.get(src, [])
        _run([hipcc, *flags, "-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
