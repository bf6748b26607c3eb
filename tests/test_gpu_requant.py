"""GPU parity of mxq_gemm_requant, the GEMM whose epilogue emits the next
layer's MX-quantized activations.

Gates, for y = act(deq(A) deq(W)^T + bias) with act none or GELU (tanh form):
  * the bf16 values y the kernel quantized (its optional bf16 output) are
    within the GEMM tolerance of the oracle's fp64 act(reference);
  * the codes and scales equal, byte for byte, the oracle's MX quantization
    of those bf16 values, and do not depend on whether y is also stored;
  * with act = none, y equals mxq_gemm's output bit for bit;
  * a chain mlp_up (GELU, requantized) -> mlp_down equals the same chain
    through a separate quantizer, bit for bit."""

import numpy as np
import pytest

import oracle
from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, bf16_bits_from_f32, make_layer_inputs
from tests._util import bf16_out_to_f64, gpu_or_skip, log_case, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _scheme(fmt):
    return {"mxfp8": oracle.MXFP8, "mxfp4": oracle.MXFP4, "mxfp6_e2m3": oracle.MXFP6_E2M3,
            "mxfp6_e3m2": oracle.MXFP6_E3M2}[fmt]


def _bits_of(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _gate(y, r):
    err = oracle.gemm_error(y, r)
    mis = oracle.rounding_mismatch_rate(y, r)
    band = int(np.sum(np.abs(r) >= np.max(np.abs(r)) / 16))
    print(f"gemm_error={err:.3e} rounding_mismatch={mis:.4f} over {band} outputs", flush=True)
    assert err <= TOL, err
    assert mis <= 0.01, mis


def _case(fmt, out_fmt, act, M, N, K, dev, seed):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    rng = np.random.default_rng(seed)
    a_bits = bf16_bits_from_f32((rng.standard_normal((M, K)) * np.exp(rng.normal(0, 0.5, (M, 1)))).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    b_bits = bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32))
    qa = mxq.quantize(fmt, to_dev(a_bits, dev))
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    bias = to_dev(b_bits, dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    q1 = mxq.gemm_requant(qa, qw, out_fmt, bias, act, out_bf16=y)
    q2 = mxq.gemm_requant(qa, qw, out_fmt, bias, act)  # without the bf16 copy
    torch.cuda.synchronize()
    return a_bits, w_bits, b_bits, qa, qw, bias, y, q1, q2


@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
@pytest.mark.parametrize("fmt,out_fmt", [("mxfp8", "mxfp8"), ("mxfp8", "mxfp4"), ("mxfp4", "mxfp8"),
                                         ("mxfp4", "mxfp4"), ("mxfp6_e2m3", "mxfp8"), ("mxfp6_e3m2", "mxfp4")])
def test_requant_matches_oracle(fmt, out_fmt, act, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    # ragged rows and a column count that is a multiple of 32 but not of the tile width
    M, N = 300, 288
    K = 512 if fmt == "mxfp4" else 256
    log_case("requant", fmt, out_fmt, act, M, N, K)
    a_bits, w_bits, b_bits, qa, qw, bias, y, q1, q2 = _case(fmt, out_fmt, act, M, N, K, dev, 41)
    ca, sa = oracle.quantize_mx(a_bits, _scheme(fmt))
    cw, sw = oracle.quantize_mx(w_bits, _scheme(fmt))
    r = oracle.gemm_mx_ref(ca, sa, cw, sw, _scheme(fmt), b_bits)
    if act == "gelu_tanh":
        r = oracle.gelu_tanh(r)
    _gate(bf16_out_to_f64(y), r)
    yc, ys = oracle.quantize_mx(_bits_of(y), _scheme(out_fmt))
    assert np.array_equal(q1.scales.cpu().numpy(), ys)
    assert np.array_equal(q1.codes.cpu().numpy(), yc)
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    if act == "none":
        assert torch.equal(y.view(torch.int16), mxq.gemm(qa, qw, bias).view(torch.int16))


def test_requant_chain_equals_separate_quantizer(dev):
    """mlp_up with GELU requantized to MXFP8, then mlp_down on those codes, equals GELU output through
    the standalone quantizer, then the same GEMM."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, D, H = 512, 256, 1024
    log_case("requant chain", M, D, H)
    rng = np.random.default_rng(43)
    x = to_dev(bf16_bits_from_f32(rng.standard_normal((M, D)).astype(np.float32)), dev)
    w_up = mxq.quantize("mxfp8", to_dev(bf16_bits_from_f32((rng.standard_normal((H, D)) * 0.05).astype(np.float32)), dev))
    w_dn = mxq.quantize("mxfp8", to_dev(bf16_bits_from_f32((rng.standard_normal((D, H)) * 0.05).astype(np.float32)), dev))
    qx = mxq.quantize("mxfp8", x)
    h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    qh = mxq.gemm_requant(qx, w_up, "mxfp8", None, "gelu_tanh", out_bf16=h)
    fused = mxq.gemm(qh, w_dn)
    separate = mxq.gemm(mxq.quantize("mxfp8", h), w_dn)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), separate.view(torch.int16))


def test_requant_nonfinite_rows(dev):
    """A NaN activation makes its output row NaN; the requantized row gets NaN scales and zero codes,
    exactly as the quantizer does on the bf16 output."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 64, 128, 256
    log_case("requant nonfinite")
    rng = np.random.default_rng(44)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[9, 17] = np.nan
    qa = mxq.quantize("mxfp8", to_dev(bf16_bits_from_f32(a), dev))
    qw = mxq.quantize("mxfp8", to_dev(bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.05).astype(np.float32)), dev))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    q = mxq.gemm_requant(qa, qw, "mxfp8", None, "none", out_bf16=y)
    torch.cuda.synchronize()
    yc, ys = oracle.quantize_mx(_bits_of(y), oracle.MXFP8)
    assert (ys[9] == 0xFF).all() and (yc[9] == 0).all()
    assert np.array_equal(q.scales.cpu().numpy(), ys) and np.array_equal(q.codes.cpu().numpy(), yc)


def test_requant_full_size_mlp_up(dev):
    """FLUX MLP up-projection (4608 x 3072 -> 12288) with GELU requantized to MXFP8 for the down-projection:
    sampled rows and columns of y against the oracle, and every code row of the sample against the oracle's
    quantization of the stored y."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    layer = WORKLOADS["flux_mlp_up_mxfp8"].layers[0]
    log_case("requant full", layer.M, layer.K, layer.N)
    a_bits, w_bits = make_layer_inputs(layer, seed=0)
    qa = mxq.quantize("mxfp8", to_dev(a_bits, dev))
    qw = mxq.quantize("mxfp8", to_dev(w_bits, dev))
    y = torch.empty((layer.M, layer.N), dtype=torch.bfloat16, device=dev)
    q = mxq.gemm_requant(qa, qw, "mxfp8", None, "gelu_tanh", out_bf16=y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(45)
    # the mismatch gate counts only outputs with |r| >= max|r| / 16; after GELU
    # that is a small share, so the sample is large enough to hold a few hundred
    rows = np.union1d(rng.choice(layer.M, 96, replace=False), [0, layer.M - 1])
    cols = np.union1d(rng.choice(layer.N, 96, replace=False), [0, layer.N - 1])
    ca, sa = oracle.quantize_mx(np.ascontiguousarray(a_bits[rows]), oracle.MXFP8)
    cw, sw = oracle.quantize_mx(np.ascontiguousarray(w_bits[cols]), oracle.MXFP8)
    r = oracle.gelu_tanh(oracle.gemm_mx_ref(ca, sa, cw, sw, oracle.MXFP8))
    ri = torch.from_numpy(rows).to(dev)
    ysel = y[ri]
    _gate(bf16_out_to_f64(ysel)[:, cols], r)
    yc, ys = oracle.quantize_mx(_bits_of(ysel), oracle.MXFP8)
    assert np.array_equal(q.codes[ri].cpu().numpy(), yc)
    assert np.array_equal(q.scales[ri].cpu().numpy(), ys)


@pytest.mark.parametrize("fmt,out_fmt,act", [("mxfp8", "mxfp8", "gelu_tanh"), ("mxfp4", "mxfp4", "none")])
def test_requant_tall_tiles_ragged(fmt, out_fmt, act, dev):
    """A shape that fits one round of 384 x 192 tiles but needs two at 256 rows (so the 384 x 192 tile is
    taken on a 256-CU device), with 4 rows and 64 columns of the last tiles empty: y in full against the
    oracle, every code and scale against the oracle's quantization of y."""
    M, N, K = 380, 49088, 256
    log_case("requant tall", fmt, out_fmt, act, M, N, K)
    a_bits, w_bits, b_bits, qa, qw, bias, y, q1, q2 = _case(fmt, out_fmt, act, M, N, K, dev, 46)
    ca, sa = oracle.quantize_mx(a_bits, _scheme(fmt))
    cw, sw = oracle.quantize_mx(w_bits, _scheme(fmt))
    r = oracle.gemm_mx_ref(ca, sa, cw, sw, _scheme(fmt), b_bits)
    if act == "gelu_tanh":
        r = oracle.gelu_tanh(r)
    _gate(bf16_out_to_f64(y), r)
    yc, ys = oracle.quantize_mx(_bits_of(y), _scheme(out_fmt))
    assert np.array_equal(q1.scales.cpu().numpy(), ys)
    assert np.array_equal(q1.codes.cpu().numpy(), yc)
    import torch

    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
