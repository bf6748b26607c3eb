"""GPU edge cases of the hot path: empty tensors, non-finite inputs, and sizes
whose element counts pass 2^31 (64-bit indexing), each against the CPU oracle
(sampled where the full result is too large for it)."""

import numpy as np
import pytest

import oracle
from microscaling_quantized_diffusion_amd.inputs import bf16_bits_from_f32
from tests._util import bf16_out_to_f64, gpu_or_skip, log_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _scheme(fmt):
    return {"mxfp8": oracle.MXFP8, "mxfp4": oracle.MXFP4}[fmt]


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_empty_tensors(fmt, dev):
    """Zero rows or zero output columns are successful no-ops (empty torch tensors have null data pointers)."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("empty", fmt)
    K = 64
    a0 = torch.empty((0, K), dtype=torch.bfloat16, device=dev)
    q0 = mxq.quantize(fmt, a0)
    assert q0.codes.shape[0] == 0 and q0.scales.shape[0] == 0
    w = to_dev(bf16_bits_from_f32(np.ones((8, K), np.float32)), dev)
    qw = mxq.quantize(fmt, w)
    out = mxq.gemm(q0, qw)
    assert tuple(out.shape) == (0, 8)
    out = mxq.quant_gemm_fused(a0, qw)
    assert tuple(out.shape) == (0, 8)
    # zero output columns: the output tensor is left untouched
    a = to_dev(bf16_bits_from_f32(np.ones((4, K), np.float32)), dev)
    qa = mxq.quantize(fmt, a)
    w0 = torch.empty((0, K), dtype=torch.bfloat16, device=dev)
    qw0 = mxq.quantize(fmt, w0)
    out = mxq.gemm(qa, qw0)
    assert tuple(out.shape) == (4, 0)
    assert tuple(mxq.gemm_bf16(a0, w).shape) == (0, 8)
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_nonfinite_activations_mx(fmt, dev):
    """A NaN or Inf in an MX block gives that block the NaN scale 0xFF: every
    output of its row is NaN, and every other output matches the oracle."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 64, 96, 256
    log_case("nonfinite mx", fmt)
    rng = np.random.default_rng(11)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[5, 10] = np.inf
    a[20, 100] = np.nan
    a[33, 255] = -np.inf
    a_bits = bf16_bits_from_f32(a)
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    out = mxq.quant_gemm_fused(to_dev(a_bits, dev), qw)
    torch.cuda.synchronize()
    y = bf16_out_to_f64(out)
    ca, sa = oracle.quantize_mx(a_bits, _scheme(fmt))
    cw, sw = oracle.quantize_mx(w_bits, _scheme(fmt))
    r = oracle.gemm_mx_ref(ca, sa, cw, sw, _scheme(fmt))
    assert np.array_equal(np.isnan(y), np.isnan(r))
    assert np.isnan(r[[5, 20, 33]]).all() and not np.isnan(np.delete(r, [5, 20, 33], axis=0)).any()
    keep = ~np.isnan(r).any(axis=1)
    err = oracle.gemm_error(y[keep], r[keep])
    assert err <= 2e-3, err


def test_nonfinite_activations_nvfp4(dev):
    """A non-finite value anywhere makes the NVFP4 tensor scale NaN, so every output is NaN."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 32, 48, 128
    log_case("nonfinite nvfp4")
    rng = np.random.default_rng(12)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[7, 3] = np.inf
    a_bits = bf16_bits_from_f32(a)
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qw = mxq.quantize("nvfp4", to_dev(w_bits, dev))
    out = mxq.quant_gemm_fused(to_dev(a_bits, dev), qw)
    torch.cuda.synchronize()
    qa = oracle.quantize_nvfp4(a_bits)
    qo = oracle.quantize_nvfp4(w_bits)
    r = oracle.gemm_nvfp4_ref(qa[0], qa[1], qa[2], qo[0], qo[1], qo[2])
    assert np.isnan(r).all()
    assert np.isnan(bf16_out_to_f64(out)).all()


def test_quantize_beyond_2g_elements(dev):
    """MXFP8 quantization of 2^31 + 2^18 elements (64-bit chunk indices); sampled rows, the last included,
    are byte-exact against the oracle."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    rows, cols = (1 << 16) + 8, 1 << 15
    log_case("quantize > 2^31 elements", rows, cols)
    g = torch.Generator(device=dev).manual_seed(21)
    x = torch.randn((rows, cols), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = mxq.quantize("mxfp8", x)
    torch.cuda.synchronize()
    pick = np.array([0, 1, 12345, (1 << 16) - 1, 1 << 16, rows - 2, rows - 1])
    bits = x[torch.from_numpy(pick).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    c, s = oracle.quantize_mx(bits, oracle.MXFP8)
    idx = torch.from_numpy(pick).to(dev)
    assert np.array_equal(q.codes[idx].cpu().numpy(), c)
    assert np.array_equal(q.scales[idx].cpu().numpy(), s)
    del x, q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K", [64, 128])
def test_gemm_output_beyond_2g_elements(K, dev):
    """An MXFP8 GEMM whose output has more than 2^31 elements (64-bit output offsets), through the
    generic tile kernel (K = 64) and the LDS-DMA kernel (K = 128); sampled rows and columns, the last
    ones included, against the oracle."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N = 49152, 46592
    log_case("gemm output > 2^31 elements", M, N, K)
    rng = np.random.default_rng(22)
    a_bits = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qa = mxq.quantize("mxfp8", to_dev(a_bits, dev))
    qw = mxq.quantize("mxfp8", to_dev(w_bits, dev))
    out = mxq.gemm(qa, qw)
    torch.cuda.synchronize()
    rows = np.union1d(rng.choice(M, 24, replace=False), [0, M - 1])
    cols = np.union1d(rng.choice(N, 24, replace=False), [0, N - 1])
    ca, sa = oracle.quantize_mx(np.ascontiguousarray(a_bits[rows]), oracle.MXFP8)
    cw, sw = oracle.quantize_mx(np.ascontiguousarray(w_bits[cols]), oracle.MXFP8)
    r = oracle.gemm_mx_ref(ca, sa, cw, sw, oracle.MXFP8)
    ri = torch.from_numpy(rows).to(dev)
    ci = torch.from_numpy(cols).to(dev)
    y = bf16_out_to_f64(out[ri][:, ci])
    err = oracle.gemm_error(y, r)
    assert err <= 2e-3, err
    del out
    torch.cuda.empty_cache()
