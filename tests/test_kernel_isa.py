"""ISA checks of the attention kernels (CPU only: hipcc cross-compiles).

A matrix-core instruction is cross-lane: a lane's result depends on operands
held by other lanes.  If the compiler moves one into a region entered under a
partial EXEC mask (e.g. the per-row store condition of the epilogue), the
disabled lanes' operands are dropped and valid rows come out wrong.  The
kernels pin their accumulators before such regions; this test checks, on the
generated gfx950 assembly, that no MFMA sits in a store's divergent region:
walking back from each global store (the O rows, the P~ / Q~ dumps, the
short-query partial states) to the nearest instruction that changes EXEC,
no MFMA may be passed when that instruction is the s_and_saveexec opening
the store's region.  It also checks that the benchmarked kernels do not
spill.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_block_quantized_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def compile_to_asm(src, tmp_path):
    from mxfp4_block_quantized_amd import build as b
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared",)] + b.EXTRA_FLAGS.get(src, [])
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip",
           os.path.join(CSRC, src), "-S", "--offload-device-only", "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def kernels(asm):
    for m in re.finditer(r"^(_Z\S*attn_\S*kernel\S*?):", asm, re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        yield name, asm[m.end():end]


def _writes_exec(t):
    op = t.split()[0]
    if op.startswith("s_and_saveexec") or op.startswith("s_or_saveexec"):
        return True
    parts = t.replace(",", " ").split()
    return op.startswith("s_") and len(parts) > 1 and parts[1] == "exec"


def mfma_in_store_regions(body):
    """MFMAs between a global store and the s_and_saveexec that opens its
    divergent region (no other EXEC change in between)."""
    lines = [l.strip() for l in body.splitlines()
             if l.strip() and not l.strip().startswith((";", ".", "//"))]
    found = []
    for i, t in enumerate(lines):
        if not t.startswith("global_store"):
            continue
        seen = []
        for u in reversed(lines[:i]):
            if _writes_exec(u):
                if u.split()[0].startswith("s_and_saveexec"):
                    found += seen
                break
            if u.startswith("v_mfma"):
                seen.append(u)
    return found


def template_args(name):
    """The integer template arguments of a mangled kernel name."""
    m = re.search(r"kernelI((?:Li-?\d+E)+)E", name)
    return [int(x) for x in re.findall(r"Li(-?\d+)E", m.group(1))] if m else []


def is_dump_variant(name):
    """The P~ dump instantiations (tests only): attn_mx_kernel<D, UOS, PNQ,
    CAUSAL, DUMP> and attn_decode_kernel<D, UOS, PNQ, DUMP, COMPACT>."""
    args = template_args(name)
    if "attn_mx_kernel" in name:
        return args[4] == 1
    if "attn_decode_kernel" in name:
        return args[3] == 1
    return False


@pytest.mark.parametrize("src", ["attn_mx.hip", "attn_f16.hip"])
def test_no_mfma_under_partial_exec(src, tmp_path):
    asm = compile_to_asm(src, tmp_path)
    found = 0
    for name, body in kernels(asm):
        found += 1
        assert not mfma_in_store_regions(body), name
    assert found > 0


@pytest.mark.parametrize("src", ["attn_mx.hip", "attn_f16.hip"])
def test_no_register_spills_in_benchmarked_kernels(src, tmp_path):
    asm = compile_to_asm(src, tmp_path)
    for name, body in kernels(asm):
        if is_dump_variant(name):
            continue  # the P~ dump variants (tests only) may spill
        m = re.search(r"ScratchSize:\s*(\d+)", body)
        if m is None:
            meta = re.search(re.escape(name) + r"[\s\S]*?\.private_segment_fixed_size:\s*(\d+)", asm)
            scratch = int(meta.group(1)) if meta else 0
        else:
            scratch = int(m.group(1))
        assert scratch == 0, (name, scratch)


def test_store_region_check_sees_a_moved_mfma():
    """The check itself: an MFMA placed between a store's s_and_saveexec and
    the store (the failure once seen) is reported; above the saveexec it is
    not."""
    bad = """
     s_and_saveexec_b64 s[4:5], vcc
     s_cbranch_execz .LBB0_2
     v_mfma_scale_f32_16x16x128_f8f6f4 v[0:3], v[4:7], v[8:11], v[0:3], v12, v13
     global_store_dwordx4 v[20:21], v[0:3], off
    .LBB0_2:
     s_or_b64 exec, exec, s[4:5]
     s_endpgm
    """
    good = bad.replace(
        "s_and_saveexec_b64 s[4:5], vcc\n     s_cbranch_execz .LBB0_2\n     v_mfma",
        "v_mfma").replace("global_store", "s_and_saveexec_b64 s[4:5], vcc\n     global_store")
    assert len(mfma_in_store_regions(bad)) == 1
    assert mfma_in_store_regions(good) == []
