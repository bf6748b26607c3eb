"""GPU parity of MXFP6 (E2M3 / E3M2 codes, E8M0 scale per 32): the quantizer byte for byte against the
oracle (every bf16 bit pattern, both shared-scale rules, ragged shapes), the GEMM within the GEMM gate
(ragged M and N, K a multiple of 128, with bias), the fused call equal to quantize + GEMM, the
slots' zero padding ignored by the MFMA, and sampled rows of the FLUX MLP up-projection."""

import numpy as np
import pytest

import oracle
from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, bf16_bits_from_f32, make_layer_inputs
from tests._util import bf16_out_to_f64, gpu_or_skip, log_case, to_dev

pytestmark = pytest.mark.gpu
FMTS = ["mxfp6_e2m3", "mxfp6_e3m2"]
TOL = 2e-3


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _scheme(fmt):
    return {"mxfp6_e2m3": oracle.MXFP6_E2M3, "mxfp6_e3m2": oracle.MXFP6_E3M2}[fmt]


def _assert_quant_same(fmt, bits, dev, rule="floor"):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    q = mxq.quantize(fmt, to_dev(bits, dev), scale_rule=rule)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_mx(bits, _scheme(fmt), rule)
    gs, gc = q.scales.cpu().numpy(), q.codes.cpu().numpy()
    bad = np.argwhere(gs != os_)
    assert bad.size == 0, f"{fmt}: {len(bad)} scale mismatches, first {bad[:3].tolist()}"
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, f"{fmt}: {len(bad)} code-byte mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("rule", ["floor", "rceil"])
@pytest.mark.parametrize("fmt", FMTS)
def test_all_bf16_patterns(fmt, rule, dev):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(64, 1024)
    log_case("mxfp6 all patterns", fmt, rule)
    _assert_quant_same(fmt, bits, dev, rule)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (129, 160), (1024, 1024)])
def test_ragged_and_activation_shapes(fmt, rows, K, dev):
    rng = np.random.default_rng(rows + K)
    x = rng.standard_normal((rows, K)) * np.exp(rng.normal(0, 2, (rows, 1)))
    log_case("mxfp6 shapes", fmt, rows, K)
    _assert_quant_same(fmt, bf16_bits_from_f32(x.astype(np.float32)), dev)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(300, 203, 256), (129, 384, 384), (64, 64, 128), (513, 1100, 640)])
def test_gemm_matches_oracle(fmt, M, N, K, dev):
    """Ragged M and N over several 256-row tiles, an odd number of 128-element K stages, bias with
    N = 203."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("mxfp6 gemm", fmt, M, N, K)
    rng = np.random.default_rng(M + N + K)
    a_bits = bf16_bits_from_f32((rng.standard_normal((M, K)) * np.exp(rng.normal(0, 0.5, (M, 1)))).astype(np.float32))
    w_bits = bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    b_bits = bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32)) if N == 203 else None
    qa = mxq.quantize(fmt, to_dev(a_bits, dev))
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    bias = None if b_bits is None else to_dev(b_bits, dev)
    y = mxq.gemm(qa, qw, bias)
    fused = mxq.quant_gemm_fused(to_dev(a_bits, dev), qw, bias)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), fused.view(torch.int16))
    ca, sa = oracle.quantize_mx(a_bits, _scheme(fmt))
    cw, sw = oracle.quantize_mx(w_bits, _scheme(fmt))
    r = oracle.gemm_mx_ref(ca, sa, cw, sw, _scheme(fmt), b_bits)
    err = oracle.gemm_error(bf16_out_to_f64(y), r)
    mis = oracle.rounding_mismatch_rate(bf16_out_to_f64(y), r)
    print(f"gemm_error={err:.3e} rounding_mismatch={mis:.4f}", flush=True)
    assert err <= TOL, err
    assert mis <= 0.01, mis


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_ignores_slot_padding(fmt, dev):
    """Bytes 24..31 of every 32-byte slot are outside the codes: filling them with ones in both
    operands leaves the GEMM's output bit for bit unchanged."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, N, K = 256, 256, 256
    log_case("mxfp6 slot padding", fmt, M, N, K)
    rng = np.random.default_rng(62)
    qa = mxq.quantize(fmt, to_dev(bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32)), dev))
    qw = mxq.quantize(fmt, to_dev(bf16_bits_from_f32((rng.standard_normal((N, K)) * 0.05).astype(np.float32)), dev))
    y = mxq.gemm(qa, qw)
    pad = torch.zeros(K, dtype=torch.bool, device=dev).view(K // 32, 32)
    pad[:, 24:] = True
    pad = pad.view(K)
    assert not bool(qa.codes[:, pad].any()) and not bool(qw.codes[:, pad].any())
    qa.codes[:, pad] = 0xFF
    qw.codes[:, pad] = 0xFF
    y2 = mxq.gemm(qa, qw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_gemm_k_not_multiple_of_128_is_unsupported(dev):
    from microscaling_quantized_diffusion_amd import mxq

    log_case("mxfp6 K % 128")
    a = to_dev(bf16_bits_from_f32(np.ones((64, 192), np.float32)), dev)
    qa = mxq.quantize("mxfp6_e2m3", a)
    with pytest.raises(mxq.MxqError) as e:
        mxq.gemm(qa, qa)
    assert e.value.status == 6


@pytest.mark.parametrize("fmt", FMTS)
def test_full_size_mlp_up(fmt, dev):
    """FLUX MLP up-projection (4608 x 3072 -> 12288) through the fused call: sampled rows and columns,
    the first and last included, against the oracle."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    layer = WORKLOADS["flux_mlp_up_mxfp8"].layers[0]
    log_case("mxfp6 full size", fmt, layer.M, layer.K, layer.N)
    a_bits, w_bits = make_layer_inputs(layer, seed=0)
    qw = mxq.quantize(fmt, to_dev(w_bits, dev))
    y = mxq.quant_gemm_fused(to_dev(a_bits, dev), qw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(61)
    rows = np.union1d(rng.choice(layer.M, 48, replace=False), [0, layer.M - 1])
    cols = np.union1d(rng.choice(layer.N, 48, replace=False), [0, layer.N - 1])
    ca, sa = oracle.quantize_mx(np.ascontiguousarray(a_bits[rows]), _scheme(fmt))
    cw, sw = oracle.quantize_mx(np.ascontiguousarray(w_bits[cols]), _scheme(fmt))
    r = oracle.gemm_mx_ref(ca, sa, cw, sw, _scheme(fmt))
    ri = torch.from_numpy(rows).to(dev)
    ci = torch.from_numpy(cols).to(dev)
    err = oracle.gemm_error(bf16_out_to_f64(y[ri][:, ci]), r)
    print(f"gemm_error={err:.3e}", flush=True)
    assert err <= TOL, err
