"""GPU checks of the packed scale layout (MXQ_SCALES_PACKED): the quantizer's packed scales are the
row-major ones permuted as include/mxq.h defines, codes unchanged; the GEMM and the fused call on packed
scales equal the row-major calls bit for bit (ragged tiles, both tile widths, every MX format); the padding
rows of the packed scales never reach a stored output."""

import numpy as np
import pytest

from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, bf16_bits_from_f32, make_layer_inputs
from tests._util import gpu_or_skip, log_case, to_dev

pytestmark = pytest.mark.gpu
P_OF = {"mxfp8": 4, "mxfp4": 8, "mxfp6_e2m3": 4, "mxfp6_e3m2": 4}  # scale blocks per row and GEMM K stage


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _packed_index(rows, S, P):
    """[rows, S] -> byte offsets of the packed layout: group r // 32, stage kb // P, row r % 32, kb % P."""
    r = np.arange(rows)[:, None]
    kb = np.arange(S)[None, :]
    return (r // 32) * 32 * S + (kb // P) * 32 * P + (r % 32) * P + kb % P


def _x(rng, rows, K, spread=1.0):
    x = rng.standard_normal((rows, K)) * np.exp(rng.normal(0, spread, (rows, 1)))
    return bf16_bits_from_f32(x.astype(np.float32))


@pytest.mark.parametrize("rule", ["floor", "rceil"])
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "mxfp6_e2m3"])
def test_quantize_packed_is_a_permutation(fmt, rule, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    rows, K = 300, 1024
    log_case("packed quantize", fmt, rule, rows, K)
    x = to_dev(_x(np.random.default_rng(71), rows, K), dev)
    qr = mxq.quantize(fmt, x, scale_rule=rule)
    qp = mxq.quantize(fmt, x, scale_rule=rule, packed_scales=True)
    torch.cuda.synchronize()
    assert qp.scales.shape == (320, K // 32)
    assert torch.equal(qp.codes, qr.codes)
    idx = _packed_index(rows, K // 32, P_OF[fmt])
    flat = qp.scales.cpu().numpy().reshape(-1)
    assert np.array_equal(flat[idx], qr.scales.cpu().numpy())


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "mxfp6_e3m2"])
@pytest.mark.parametrize("M,N,K", [(300, 288, 512), (513, 1100, 1024), (64, 96, 256)])
def test_gemm_packed_equals_row_major(fmt, M, N, K, dev):
    """Bit for bit, with the packed scales' padding rows set to the NaN scale 0xFF."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("packed gemm", fmt, M, N, K)
    rng = np.random.default_rng(M + N + K)
    a = to_dev(_x(rng, M, K), dev)
    w = to_dev(bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.05).astype(np.float32)), dev)
    bias = to_dev(bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32)), dev)
    qa, qw = mxq.quantize(fmt, a), mxq.quantize(fmt, w)
    pa, pw = mxq.quantize(fmt, a, packed_scales=True), mxq.quantize(fmt, w, packed_scales=True)
    for q, rows in ((pa, M), (pw, N)):  # padding rows: whole 32-row groups past the last row
        flat = q.scales.view(-1)
        S = K // 32
        pad = torch.from_numpy(np.setdiff1d(np.arange(flat.numel()), _packed_index(rows, S, P_OF[fmt]).reshape(-1)))
        flat[pad.to(dev)] = 0xFF
    y = mxq.gemm(qa, qw, bias)
    yp = mxq.gemm(pa, pw, bias)
    f = mxq.quant_gemm_fused(a, qw, bias)
    fp = mxq.quant_gemm_fused(a, pw, bias)
    torch.cuda.synchronize()
    assert torch.equal(yp.view(torch.int16), y.view(torch.int16))
    assert torch.equal(fp.view(torch.int16), f.view(torch.int16))
    assert torch.equal(f.view(torch.int16), y.view(torch.int16))


def test_packed_full_size_mlp_up(dev):
    """FLUX MLP up-projection (4608 x 3072 -> 12288, the 256 x 320 tile): the fused call on packed weight
    scales equals the row-major one over the whole output."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    layer = WORKLOADS["flux_mlp_up_mxfp8"].layers[0]
    log_case("packed full size", layer.M, layer.K, layer.N)
    a_bits, w_bits = make_layer_inputs(layer, seed=0)
    a, w = to_dev(a_bits, dev), to_dev(w_bits, dev)
    y = mxq.quant_gemm_fused(a, mxq.quantize("mxfp8", w))
    yp = mxq.quant_gemm_fused(a, mxq.quantize("mxfp8", w, packed_scales=True))
    torch.cuda.synchronize()
    assert torch.equal(yp.view(torch.int16), y.view(torch.int16))


def test_mixed_layouts_rejected(dev):
    from microscaling_quantized_diffusion_amd import mxq

    log_case("packed mixed layouts")
    x = to_dev(_x(np.random.default_rng(72), 64, 256), dev)
    qa, pw = mxq.quantize("mxfp8", x), mxq.quantize("mxfp8", x, packed_scales=True)
    with pytest.raises(ValueError):
        mxq.gemm(qa, pw)
    with pytest.raises(ValueError):
        mxq.gemm_requant(qa, pw, "mxfp8")
