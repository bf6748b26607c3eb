"""GPU parity of producer-fused quantization into a concatenated activation.

A FLUX single-stream block feeds its output projection (linear2) with the
concatenation of the attention output and the GELU of the MLP part of
linear1.  Both producers can emit their MX codes straight into that
concatenated matrix: the requantizing GEMM and the requantizing attention write
column slices of a wider code / scale matrix (row strides).  Gates, all bit for
bit: each producer equals its unfused path (bf16 output, then the standalone
quantizer); bytes outside the slice are untouched; linear2 on the fused
concatenation equals linear2 on the unfused one.
"""

import numpy as np
import pytest

from microscaling_quantized_diffusion_amd.inputs import bf16_bits_from_f32
from tests._util import gpu_or_skip, log_case, to_dev

pytestmark = pytest.mark.gpu
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _bf16(rng, shape, scale, dev):
    return to_dev(bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32).reshape(-1, shape[-1]))
                  .reshape(shape), dev)


def _wide(fmt, rows, cols, dev):
    """A sentinel-filled quantized matrix [rows, cols] (codes and scales)."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    codes = torch.full((rows, mxq.code_cols(fmt, cols)), SENTINEL, dtype=torch.uint8, device=dev)
    scales = torch.full((rows, cols // 32), SENTINEL, dtype=torch.uint8, device=dev)
    return mxq.QTensor(fmt, codes, scales, None, cols)


def _slice(q, c0, c1):
    """Columns [c0, c1) of a quantized matrix as a strided view."""
    from microscaling_quantized_diffusion_amd import mxq

    b = 1 if q.fmt == "mxfp8" else 2
    return mxq.QTensor(q.fmt, q.codes[:, c0 // b:c1 // b], q.scales[:, c0 // 32:c1 // 32], None, c1 - c0)


def _outside_untouched(q, c0, c1):
    import torch

    b = 1 if q.fmt == "mxfp8" else 2
    for t, lo, hi in ((q.codes, c0 // b, c1 // b), (q.scales, c0 // 32, c1 // 32)):
        mask = torch.ones(t.shape[1], dtype=torch.bool, device=t.device)
        mask[lo:hi] = False
        assert bool((t[:, mask] == SENTINEL).all())


@pytest.mark.parametrize("out_fmt", ["mxfp8", "mxfp4"])
def test_gemm_requant_into_column_slice(out_fmt, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K, c0, wide = 300, 288, 256, 96, 640
    log_case("gemm requant slice", out_fmt, M, N, K, c0)
    rng = np.random.default_rng(51)
    qa = mxq.quantize("mxfp8", _bf16(rng, (M, K), 1.0, dev))
    qw = mxq.quantize("mxfp8", _bf16(rng, (N, K), 0.05, dev))
    dense = mxq.gemm_requant(qa, qw, out_fmt, None, "gelu_tanh")
    big = _wide(out_fmt, M, wide, dev)
    mxq.gemm_requant(qa, qw, out_fmt, None, "gelu_tanh", out=_slice(big, c0, c0 + N))
    torch.cuda.synchronize()
    s = _slice(big, c0, c0 + N)
    assert torch.equal(s.codes, dense.codes) and torch.equal(s.scales, dense.scales)
    _outside_untouched(big, c0, c0 + N)


@pytest.mark.parametrize("out_fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("B,H,S", [(1, 2, 256), (2, 3, 320)])
def test_attention_requant_matches_quantized_output(out_fmt, B, H, S, dev):
    """The requantized attention output equals attention_fp8's bf16 output, laid out token-major
    (heads side by side) and quantized by the standalone quantizer."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("attention requant", out_fmt, B, H, S)
    rng = np.random.default_rng(52 + S)
    q, k, v = (_bf16(rng, (B, H, S, 128), 1.0, dev) for _ in range(3))
    o = mxq.attention_fp8(q, k, v)
    want = mxq.quantize(out_fmt, o.permute(0, 2, 1, 3).reshape(B * S, H * 128).contiguous())
    got = mxq.attention_fp8_requant(q, k, v, out_fmt)
    torch.cuda.synchronize()
    assert torch.equal(got.scales, want.scales)
    assert torch.equal(got.codes, want.codes)


def test_attention_requant_into_column_slice(dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    B, H, S, c0, wide = 1, 2, 192, 64, 512
    log_case("attention requant slice", B, H, S, c0)
    rng = np.random.default_rng(53)
    q, k, v = (_bf16(rng, (B, H, S, 128), 1.0, dev) for _ in range(3))
    dense = mxq.attention_fp8_requant(q, k, v, "mxfp4")
    big = _wide("mxfp4", B * S, wide, dev)
    mxq.attention_fp8_requant(q, k, v, "mxfp4", out=_slice(big, c0, c0 + H * 128))
    torch.cuda.synchronize()
    s = _slice(big, c0, c0 + H * 128)
    assert torch.equal(s.codes, dense.codes) and torch.equal(s.scales, dense.scales)
    _outside_untouched(big, c0, c0 + H * 128)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_single_block_concat_chain(fmt, dev):
    """A single-stream block's linear2 input built by the producers' epilogues equals the one built
    through bf16 and the standalone quantizer, and so does linear2's output, bit for bit: attention
    codes in columns [0, D), GELU(MLP part of linear1) codes in [D, D + F)."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    B, H, S, F = 1, 2, 256, 1024
    D = H * 128
    M = B * S
    log_case("single block concat", fmt, B, H, S, F)
    rng = np.random.default_rng(54)
    q, k, v = (_bf16(rng, (B, H, S, 128), 1.0, dev) for _ in range(3))
    x = mxq.quantize(fmt, _bf16(rng, (M, D), 1.0, dev))
    w_mlp = mxq.quantize(fmt, _bf16(rng, (F, D), 0.05, dev))
    w2 = mxq.quantize(fmt, _bf16(rng, (D, D + F), 0.03, dev))
    # fused: both producers write their codes into the concatenation
    cat = _wide(fmt, M, D + F, dev)
    mxq.attention_fp8_requant(q, k, v, fmt, out=_slice(cat, 0, D))
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    mxq.gemm_requant(x, w_mlp, fmt, None, "gelu_tanh", out=_slice(cat, D, D + F), out_bf16=h)
    y_fused = mxq.gemm(cat, w2)
    # unfused: bf16 producers, concatenation in bf16, the standalone quantizer
    o = mxq.attention_fp8(q, k, v).permute(0, 2, 1, 3).reshape(M, D)
    cat_ref = mxq.quantize(fmt, torch.cat([o, h], dim=1).contiguous())
    y_ref = mxq.gemm(cat_ref, w2)
    torch.cuda.synchronize()
    assert torch.equal(cat.codes, cat_ref.codes) and torch.equal(cat.scales, cat_ref.scales)
    assert torch.equal(y_fused.view(torch.int16), y_ref.view(torch.int16))
