"""GPU parity of the block quantizer, transposed quantizer and dequantizer:
codes and E8M0 bytes bit-exact against the oracle."""
import numpy as np
import pytest

from common import RULE_IDS, gpu, mxsynth, np_u8, oracle, to_torch

pytestmark = pytest.mark.gpu


def _edge_blocks():
    f32 = np.float32
    blocks = [
        np.zeros(32, f32), -np.zeros(32, f32),
        np.r_[f32(7.25), np.zeros(31, f32)],
        np.r_[np.nextafter(f32(7.25), f32(8)), np.zeros(31, f32)],
        np.r_[np.nextafter(f32(8), f32(0)), np.zeros(31, f32)],
        np.r_[f32(-1e-40), np.full(31, f32(1e-45))],
        np.r_[f32(3e-39), np.full(31, f32(-2e-39))],
        np.full(32, np.finfo(f32).max), np.full(32, -np.finfo(f32).max),
        np.r_[f32(1.0), np.full(31, f32(-0.001))],
        np.linspace(-6, 6, 32).astype(f32),
        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, f32),
        np.array([-0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -7.0] * 4, f32),
    ]
    rng = np.random.default_rng(7)
    for k in (-140, -127, -126, -60, 0, 60, 120):
        for base in (1.0, 1.8125, 7.25, 3.625):
            blk = (rng.uniform(-1, 1, 32) * base * 2.0 ** k).astype(f32)
            blk[rng.integers(32)] = f32(base * 2.0 ** k)
            blocks.append(blk)
    return np.concatenate(blocks)


@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_tiny_quant_fp32(rule):
    torch, mx = gpu()
    x = mxsynth.tiny_quant(1)
    c, s = mx.quantize(to_torch(x), rule)
    rc, rs = oracle.quantize(x, RULE_IDS[rule])
    assert np.array_equal(np_u8(c), rc)
    assert np.array_equal(np_u8(s), rs)


@pytest.mark.parametrize("rule", ["ocp", "uos"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_edge_blocks(rule, dt):
    torch, mx = gpu()
    x = _edge_blocks()
    if dt == "bf16":
        x = mxsynth.f32_to_bf16_bits(x)
        # fp32 max rounds to bf16 infinity; inputs must be finite, so use
        # the largest finite bf16 magnitude there
        x[(x & 0x7FFF) == 0x7F80] -= 1
    c, s = mx.quantize(to_torch(x), rule)
    rc, rs = oracle.quantize(x, RULE_IDS[rule])
    assert np.array_equal(np_u8(s), rs)
    assert np.array_equal(np_u8(c), rc)


@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_every_bf16_value(rule):
    """All finite bf16 patterns, in blocks sorted by magnitude and shuffled."""
    torch, mx = gpu()
    bits = np.r_[np.arange(0, 0x7F80), np.arange(0x8000, 0xFF80)].astype(np.uint16)
    bits = np.r_[bits, bits[: (-bits.size) % 32]]
    rng = np.random.default_rng(1)
    for arr in (bits, rng.permutation(bits)):
        c, s = mx.quantize(to_torch(arr), rule)
        rc, rs = oracle.quantize(arr, RULE_IDS[rule])
        assert np.array_equal(np_u8(s), rs)
        assert np.array_equal(np_u8(c), rc)


@pytest.mark.parametrize("rule", ["ocp", "uos"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 57, 64), (3, 300, 128), (2, 32, 40), (1, 1, 128)])
def test_quantize_t(rule, dt, shape):
    torch, mx = gpu()
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * 3).astype(np.float32)
    if dt == "bf16":
        x = mxsynth.f32_to_bf16_bits(x)
    c, s = mx.quantize_t(to_torch(x), rule)
    c, s = np_u8(c), np_u8(s)
    for b in range(shape[0]):
        rc, rs = oracle.quantize_t(x[b], RULE_IDS[rule])
        assert np.array_equal(c[b], rc)
        assert np.array_equal(s[b], rs)


def test_quantize_t_padded_rows():
    """rows_pad beyond ceil32(rows): extra blocks are zero codes, X = 0."""
    torch, mx = gpu()
    x = np.random.default_rng(3).standard_normal((2, 70, 128)).astype(np.float32)
    c, s = mx.quantize_t(to_torch(x), "uos", rows_pad=256)
    c, s = np_u8(c), np_u8(s)
    for b in range(2):
        rc, rs = oracle.quantize_t(x[b], oracle.RULE_UOS)
        assert np.array_equal(c[b][:, :48], rc) and np.all(c[b][:, 48:] == 0)
        assert np.array_equal(s[b][:, :3], rs) and np.all(s[b][:, 3:] == 0)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_all_codes_all_scales(out):
    torch, mx = gpu()
    codes = np.arange(16, dtype=np.uint8)
    packed = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), 2)  # 32 elements
    X = np.arange(256, dtype=np.uint8)
    allc = np.tile(packed, 256)
    y = mx.dequantize(to_torch(allc), to_torch(X),
                      torch.float32 if out == "f32" else torch.bfloat16)
    y = y.float().cpu().numpy()
    ref = oracle.dequantize(allc, X)
    with np.errstate(over="ignore"):
        ref32 = ref.astype(np.float32)
    ok = X.repeat(32) < 255
    assert np.array_equal(y[ok], ref32[ok])
    assert np.all(np.isnan(y[~ok]))  # E8M0 255 is NaN


def test_roundtrip_full_size():
    """The 8192 x 28672 bf16 roundtrip tensor: codes and scales bit-exact in
    both modes, dequantized values exact, UOS relative Frobenius error no
    worse than OCP's."""
    torch, mx = gpu()
    x = mxsynth.roundtrip_tensor(2)
    xt = to_torch(x)
    errs = {}
    for rule in ("ocp", "uos"):
        c, s = mx.quantize(xt, rule)
        rc, rs = oracle.quantize(x, RULE_IDS[rule])
        assert np.array_equal(np_u8(s), rs)
        assert np.array_equal(np_u8(c), rc)
        y = mx.dequantize(c, s, torch.float32)
        xf = xt.float().reshape(-1)
        errs[rule] = (torch.linalg.vector_norm((xf - y).double()) /
                      torch.linalg.vector_norm(xf.double())).item()
        # spot-check dequantized values against the oracle
        idx = np.random.default_rng(0).integers(0, x.size // 32, 2000)
        ref = oracle.dequantize(rc.reshape(-1, 16)[idx], rs[idx])
        got = y.reshape(-1, 32)[torch.from_numpy(idx).cuda()].reshape(-1).cpu().numpy()
        assert np.array_equal(got, ref.astype(np.float32))
    assert errs["uos"] <= errs["ocp"] < 0.2
