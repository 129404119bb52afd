"""The Python binding's argument checks: tensors the C ABI would read or
write as raw device memory are validated first (device, contiguity, dtype,
shapes, buffer sizes), so a misuse raises instead of reading or writing out
of bounds.  Every case raises before any library call."""
import pytest

from common import gpu

pytestmark = pytest.mark.gpu


def test_attention_arguments():
    torch, mx = gpu()
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 96, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):  # host tensor
        mx.attn_fwd(q.cpu(), k, k)
    with pytest.raises(TypeError):  # k in another dtype than q
        mx.attn_fwd(q, k.float(), k)
    with pytest.raises(ValueError):  # not contiguous
        mx.attn_fwd(q.transpose(2, 3), k, k)
    with pytest.raises(ValueError):  # v shape differs from k
        mx.attn_fwd(q, k, k[:, :, :64])
    with pytest.raises(ValueError):  # head dims differ
        mx.attn_fwd(q, k[..., :32].contiguous(), k[..., :32].contiguous())
    with pytest.raises(ValueError):  # output of the wrong shape
        mx.attn_fwd(q, k, k, out=torch.empty((1, 2, 63, 64), device="cuda"))
    with pytest.raises(TypeError):  # output not fp32
        mx.attn_fwd(q, k, k, out=torch.empty((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):  # workspace not bytes
        mx.attn_fwd(q, k, k, workspace=torch.empty(1 << 20, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):  # dump rows out of range
        mx.attn_fwd_dump(q, k, k, [0, 1 * 2 * 64])
    with pytest.raises(ValueError):  # lengths of another batch size
        mx.attn_fwd_varlen(q, k, k, [64, 64], [96])
    with pytest.raises(ValueError):
        mx.attn_decode_varlen(q[:, :, :1].contiguous(), k, k, [96, 1])


def test_quantizer_and_gemm_arguments():
    torch, mx = gpu()
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # codes buffer too small
        mx.quantize(x, "uos", torch.empty(100, dtype=torch.uint8, device="cuda"))
    with pytest.raises(TypeError):  # scales buffer of another dtype
        mx.quantize(x, "uos", None, torch.empty(16, dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        mx.quantize(x.cpu(), "uos")
    c, s = mx.quantize(x, "uos")
    with pytest.raises(ValueError):  # too few scale bytes for the codes
        mx.dequantize(c, s[:4])
    with pytest.raises(ValueError):  # output too small
        mx.dequantize(c, s, out=torch.empty(100, device="cuda"))
    w = torch.zeros((256, 128), dtype=torch.bfloat16, device="cuda")
    wc, ws = mx.quantize(w, "uos")
    with pytest.raises(ValueError):  # a holds fewer rows than M says
        mx.gemm(c, s, wc, ws, 8, 256, 128)
    with pytest.raises(ValueError):  # output too small
        mx.gemm(c, s, wc, ws, 4, 256, 128, out=torch.empty((4, 255), device="cuda"))
    with pytest.raises(ValueError):
        mx.linear_w4a4(x.reshape(-1), wc, ws, 256)
