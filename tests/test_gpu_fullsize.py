"""Full-tensor parity at the FLUX workload sizes, through the calls the benchmark times.

Every layer of the five workloads (and the MXFP6 variant of the MLP up-projection) runs at its real size:
  * quantized layers go through mxq_quant_gemm_fused with the weights pre-quantized as the benchmark
    does (MX scales in the packed layout); the activation codes and scales the call left in its
    workspace, the weight codes and scales, and (NVFP4) both tensor scales equal the oracle's
    quantization byte for byte over every row;
  * every output is gated against the oracle's fp64 reference from the oracle's own codes: the 2e-3
    normwise bound beyond the bf16 output rounding, the same bound per row against that row's own
    max|r|, and at most 1 % nearest-even rounding mismatches among the large outputs;
  * the double-stream block (batch 1 and 4) runs as one HIP-graph replay of its five linears (the
    modulation linear falls back to bf16 by the min(M, K, N) < 1024 rule), after eager library work
    on other buffers and with the outputs cleared; each replay equals the eager run bit for bit, and
    the replayed outputs are the ones gated against the oracle.
The oracle's quantizer runs on row chunks in a thread pool (tests._util.oracle_rows); the oracle itself
is unchanged."""

import numpy as np
import pytest

import oracle
from microscaling_quantized_diffusion_amd.inputs import WORKLOADS, make_layer_inputs
from tests._util import (bf16_out_to_f64, fused_workspace_a, gpu_or_skip, log_case, oracle_rows,
                         row_major_scales, to_dev)

pytestmark = pytest.mark.gpu
TOL = 2e-3
MISMATCH = 0.01
SCHEME = {"mxfp8": oracle.MXFP8, "mxfp4": oracle.MXFP4, "mxfp6_e2m3": oracle.MXFP6_E2M3,
          "mxfp6_e3m2": oracle.MXFP6_E3M2}


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _gate(y, r):
    err = oracle.gemm_error(y, r)
    rows = oracle.gemm_error_rows(y, r)
    mis = oracle.rounding_mismatch_rate(y, r)
    print(f"outputs={r.size} gemm_error={err:.3e} per_row={rows:.3e} rounding_mismatch={mis:.4f}", flush=True)
    assert err <= TOL, err
    assert rows <= TOL, rows
    assert mis <= MISMATCH, mis


def _oracle_quant(fmt, bits, ts=None):
    if fmt == "nvfp4":
        return oracle_rows(oracle.quantize_nvfp4, bits, ts)
    return oracle_rows(oracle.quantize_mx, bits, SCHEME[fmt]) + (None,)


def _oracle_ref(fmt, qa, qw):
    if fmt == "nvfp4":
        return oracle.gemm_nvfp4_ref(qa[0], qa[1], qa[2], qw[0], qw[1], qw[2])
    return oracle.gemm_mx_ref(qa[0], qa[1], qw[0], qw[1], SCHEME[fmt])


def _check_bytes(name, got, want):
    assert got.shape == want.shape, (name, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{name}: {bad.size} bytes differ, first at flat index {bad[0]}"


def _check_layer(fmt, M, K, a_bits, w_bits, qw, ws, out):
    """Codes, scales and tensor scales of both operands byte for byte; the whole output gated."""
    ts_a = ts_w = None
    if fmt == "nvfp4":
        ts_a, ts_w = oracle.nvfp4_tensor_scale(a_bits), oracle.nvfp4_tensor_scale(w_bits)
    oqa, oqw = _oracle_quant(fmt, a_bits, ts_a), _oracle_quant(fmt, w_bits, ts_w)
    packed = fmt != "nvfp4"
    ac, asc = fused_workspace_a(fmt, M, K, ws, packed)
    _check_bytes("A codes", ac, oqa[0])
    _check_bytes("A scales", asc, oqa[1])
    _check_bytes("W codes", qw.codes.cpu().numpy(), oqw[0])
    _check_bytes("W scales", row_major_scales(qw), oqw[1])
    if fmt == "nvfp4":
        cb, sb = M * K // 2, M * K // 16
        t0 = (cb + 255) // 256 * 256 + (sb + 255) // 256 * 256
        ts_dev = ws[t0:t0 + 4].cpu().numpy().view(np.float32)[0]
        assert ts_dev == np.float32(oqa[2]), (ts_dev, oqa[2])
        assert np.float32(qw.tensor_scale.cpu().numpy()[0]) == np.float32(oqw[2])
    _gate(bf16_out_to_f64(out), _oracle_ref(fmt, oqa, oqw))


LAYERS = [(wl, li) for wl in ("mxfp8_1024", "flux_mlp_up_mxfp8", "flux_mlp_up_mxfp6", "flux_single_mxfp4",
                              "flux_2048_nvfp4") for li in range(len(WORKLOADS[wl].layers))]


@pytest.mark.parametrize("workload,li", LAYERS, ids=[f"{w}-{WORKLOADS[w].layers[i].name}" for w, i in LAYERS])
def test_full_size_layer(workload, li, dev):
    """One fused quantize + GEMM call at the layer's full size, exactly as the benchmark issues it."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    layer = WORKLOADS[workload].layers[li]
    M, K, N, fmt = layer.M, layer.K, layer.N, layer.fmt
    log_case("fullsize", workload, layer.name, M, K, N, fmt)
    a_bits, w_bits = make_layer_inputs(layer, seed=li)
    a = to_dev(a_bits, dev)
    qw = mxq.quantize(fmt, to_dev(w_bits, dev), packed_scales=fmt != "nvfp4")
    ws = torch.empty(mxq.workspace_bytes(fmt, M, K, True), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    mxq.quant_gemm_fused(a, qw, None, out, ws)
    torch.cuda.synchronize()
    _check_layer(fmt, M, K, a_bits, w_bits, qw, ws, out)
    del a, qw, ws, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [1, 4])
def test_full_size_block_graphed(batch, dev):
    """The double-stream block's five linears as one HIP-graph replay, every output against the oracle."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    layers = WORKLOADS[f"flux_double_block_b{batch}"].layers
    bits, lins, inputs = [], [], []
    for li, layer in enumerate(layers):
        a_bits, w_bits = make_layer_inputs(layer, seed=li)
        bits.append((a_bits, w_bits))
        quantized = mxq.should_quantize(layer.M, layer.K, layer.N)
        lins.append(mxq.QuantLinear.from_weight(layer.fmt, to_dev(w_bits, dev), quantize_weight=quantized))
        inputs.append(to_dev(a_bits, dev))
    seq = mxq.LinearSequence(lins, inputs)
    eager = [o.clone() for o in seq()]
    torch.cuda.synchronize()
    graph = mxq.GraphedCall(seq)
    other = mxq.LinearSequence(lins, [x.clone() for x in inputs])
    for rep in range(2):
        log_case("block graph replay", batch, rep)
        for o in seq.outs:
            o.zero_()
        other()
        graph()
        torch.cuda.synchronize()
        for o, e in zip(seq.outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), rep
    for li, layer in enumerate(layers):
        log_case("block layer", batch, layer.name, layer.M, layer.K, layer.N)
        a_bits, w_bits = bits[li]
        if mxq.should_quantize(layer.M, layer.K, layer.N):
            _check_layer(layer.fmt, layer.M, layer.K, a_bits, w_bits, lins[li].qweight, seq.workspaces[li],
                         seq.outs[li])
        else:
            assert layer.name == "modulation"
            _gate(bf16_out_to_f64(seq.outs[li]), oracle.gemm_bf16_ref(a_bits, w_bits))
    del seq, other, graph, lins, inputs, eager
    torch.cuda.empty_cache()
