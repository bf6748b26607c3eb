"""GPU parity of the GEMM entry points against the CPU oracle.

Small and ragged shapes (several tiles plus partial ones) are compared in full
here; the FLUX-shaped workloads are compared in full at their real sizes in
test_gpu_fullsize.py.  Gates, against
the fp64 reference r computed from the oracle's own codes:
  * codes, scales and tensor scales byte-exact;
  * max_i (|y_i - r_i| - halfulp_bf16(y_i))+ / max|r| <= 2e-3, i.e. the 2e-3
    normwise bound on the result before its bf16 output rounding (that
    rounding alone may reach 2^-8 = 3.9e-3 of max|r|), and the same bound per
    row against that row's own max|r|;
  * at most 1% of the outputs with |r_i| >= max|r|/16 differ from the
    nearest-even bf16 rounding of r_i (a truncating epilogue fails this)."""

import numpy as np
import pytest

import oracle
from microscaling_quantized_diffusion_amd.inputs import bf16_bits_from_f32
from tests._util import bf16_out_to_f64, gpu_or_skip, log_case, row_major_scales, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3
MISMATCH = 0.01


def _gate(y, r):
    err = oracle.gemm_error(y, r)
    rows = oracle.gemm_error_rows(y, r)
    mis = oracle.rounding_mismatch_rate(y, r)
    raw = oracle.normwise_error(y, r)
    print(f"gemm_error={err:.3e} per_row={rows:.3e} raw_normwise={raw:.3e} rounding_mismatch={mis:.4f}", flush=True)
    assert err <= TOL, err
    assert rows <= TOL, rows
    assert mis <= MISMATCH, mis


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _scheme(fmt):
    return {"mxfp8": oracle.MXFP8, "mxfp4": oracle.MXFP4}[fmt]


def _oracle_q(fmt, bits, ts=None):
    if fmt == "nvfp4":
        return oracle.quantize_nvfp4(bits, ts)
    c, s = oracle.quantize_mx(bits, _scheme(fmt))
    return c, s, None


def _oracle_ref(fmt, qa, qw, bias=None):
    if fmt == "nvfp4":
        return oracle.gemm_nvfp4_ref(qa[0], qa[1], qa[2], qw[0], qw[1], qw[2], bias)
    return oracle.gemm_mx_ref(qa[0], qa[1], qw[0], qw[1], _scheme(fmt), bias)


def _check_q(fmt, q, oq, rows=None):
    c, s = q.codes.cpu().numpy(), row_major_scales(q)
    if rows is not None:
        c, s = c[rows], s[rows]
    assert np.array_equal(s, oq[1]), f"{fmt} scales differ"
    assert np.array_equal(c, oq[0]), f"{fmt} codes differ"
    if fmt == "nvfp4":
        assert np.float32(q.tensor_scale.cpu().numpy()[0]) == np.float32(oq[2])


SHAPES = [(1, 1, 32), (37, 45, 96), (128, 128, 256), (300, 260, 1024), (129, 64, 4096), (16, 300, 64)]


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_shapes(fmt, M, N, K, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("gemm", fmt, M, N, K)
    rng = np.random.default_rng(M * 1000 + N + K)
    a_bits = bf16_bits_from_f32((rng.standard_normal((M, K)) * np.exp(rng.normal(0, 0.5, (M, 1)))).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qa = mxq.quantize(fmt, to_dev(a_bits, dev))
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    out = mxq.gemm(qa, qw)
    torch.cuda.synchronize()
    oqa, oqw = _oracle_q(fmt, a_bits), _oracle_q(fmt, w_bits)
    _check_q(fmt, qa, oqa)
    _check_q(fmt, qw, oqw)
    _gate(bf16_out_to_f64(out), _oracle_ref(fmt, oqa, oqw))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_gemm_bias_and_fused_identity(fmt, dev):
    """Bias is added in fp32 before rounding; the fused call equals quantize + gemm bit for bit."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 200, 136, 512
    log_case("gemm bias/fused", fmt)
    rng = np.random.default_rng(99)
    a_bits = bf16_bits_from_f32(rng.standard_t(4, (M, K)).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b_bits = bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32))
    a, bias = to_dev(a_bits, dev), to_dev(b_bits, dev)
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    qa = mxq.quantize(fmt, a)
    out1 = mxq.gemm(qa, qw, bias)
    out2 = mxq.quant_gemm_fused(a, qw, bias)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    oqa, oqw = _oracle_q(fmt, a_bits), _oracle_q(fmt, w_bits)
    _gate(bf16_out_to_f64(out2), _oracle_ref(fmt, oqa, oqw, b_bits))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_gemm_wide_tiles_ragged(fmt, dev):
    """A shape whose tiles fill a second round at 256 columns but one round at
    320 (so the 256 x 320 tile is taken on a 256-CU device), with ragged rows
    and a ragged last column of tiles, compared in full."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 250, 65590, 256
    log_case("gemm wide", fmt, M, N, K)
    rng = np.random.default_rng(7)
    a_bits = bf16_bits_from_f32((rng.standard_normal((M, K)) * np.exp(rng.normal(0, 0.5, (M, 1)))).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    qa = mxq.quantize(fmt, to_dev(a_bits, dev))
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    out = mxq.gemm(qa, qw)
    torch.cuda.synchronize()
    oqa, oqw = _oracle_q(fmt, a_bits), _oracle_q(fmt, w_bits)
    _gate(bf16_out_to_f64(out), _oracle_ref(fmt, oqa, oqw))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_gemm_tall_tiles_ragged(fmt, dev):
    """A shape that fits one round of 384 x 192 tiles but needs two at 256 rows
    (so the 384 x 192 tile is taken on a 256-CU device), with 4 rows and 52
    columns of the last tiles empty, compared in full; the packed scale layout
    gives the same output bit for bit."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 380, 49100, 256
    log_case("gemm tall", fmt, M, N, K)
    rng = np.random.default_rng(11)
    a_bits = bf16_bits_from_f32((rng.standard_normal((M, K)) * np.exp(rng.normal(0, 0.5, (M, 1)))).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    a, w = to_dev(a_bits, dev), to_dev(w_bits, dev)
    qa, qw = mxq.quantize(fmt, a), mxq.quantize(fmt, w)
    out = mxq.gemm(qa, qw)
    out_p = mxq.gemm(mxq.quantize(fmt, a, packed_scales=True), mxq.quantize(fmt, w, packed_scales=True))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_p.view(torch.int16))
    oqa, oqw = _oracle_q(fmt, a_bits), _oracle_q(fmt, w_bits)
    _gate(bf16_out_to_f64(out), _oracle_ref(fmt, oqa, oqw))


def test_identity_weights(dev):
    """W = I reproduces bf16(dequant(A)) exactly (one nonzero product per output)."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    K = 256
    rng = np.random.default_rng(5)
    a_bits = bf16_bits_from_f32(rng.standard_normal((64, K)).astype(np.float32))
    eye = bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    for fmt in ("mxfp8", "mxfp4"):
        out = mxq.quant_gemm_fused(to_dev(a_bits, dev), mxq.quantize(fmt, to_dev(eye, dev)))
        torch.cuda.synchronize()
        c, s, _ = _oracle_q(fmt, a_bits)
        want = oracle.dequant_mx(c, s, _scheme(fmt))
        assert np.array_equal(bf16_out_to_f64(out), want), fmt


BF16_SHAPES = [(1, 18432, 3072), (4, 18432, 3072), (16, 512, 1024), (37, 300, 64), (200, 260, 1024), (5, 7, 40),
               (300, 200, 40), (1, 1, 8),
               # the skinny W stream at 5..16 rows: a ragged N, the modulation shape, and 128 KiB of activations
               (5, 1001, 3072), (13, 777, 1024), (8, 18432, 3072), (16, 18432, 3072), (16, 1000, 4096),
               (17, 300, 1024)]


@pytest.mark.parametrize("M,N,K", BF16_SHAPES)
def test_bf16_gemm(M, N, K, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("bf16", M, N, K)
    rng = np.random.default_rng(M + N + K)
    a_bits = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    b_bits = bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32))
    out = mxq.gemm_bf16(to_dev(a_bits, dev), to_dev(w_bits, dev), to_dev(b_bits, dev))
    torch.cuda.synchronize()
    _gate(bf16_out_to_f64(out), oracle.gemm_bf16_ref(a_bits, w_bits, b_bits))
