"""HIP-graph capture of a DiT block's linear sequence (selective quantization
included): every replay equals the eager run bit for bit, with eager library
work and new input contents between replays."""

import numpy as np
import pytest

from microscaling_quantized_diffusion_amd.inputs import bf16_bits_from_f32
from tests._util import gpu_or_skip, log_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _bits(rng, shape, scale=1.0):
    return bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_graph_replays_equal_eager(fmt, dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    log_case("graph", fmt)
    rng = np.random.default_rng(31)
    # (M, K, N): three quantized linears and one that falls back to bf16 (M = 2)
    shapes = [(1024, 1024, 2048), (1024, 2048, 1024), (1152, 1024, 1280), (2, 1024, 3072)]
    layers, inputs = [], []
    for M, K, N in shapes:
        w = to_dev(_bits(rng, (N, K), 0.02), dev)
        layers.append(mxq.QuantLinear.from_weight(fmt, w, to_dev(_bits(rng, (N,)), dev)))
        inputs.append(to_dev(_bits(rng, (M, K)), dev))
    seq = mxq.LinearSequence(layers, inputs)
    ref = [o.clone() for o in seq()]
    torch.cuda.synchronize()
    g = mxq.GraphedCall(seq)
    # eager work from the same library on other buffers between replays
    other = mxq.LinearSequence(layers, [x.clone() for x in inputs])
    for r in range(3):
        for o in seq.outs:
            o.zero_()
        other()
        g()
        torch.cuda.synchronize()
        for got, want in zip(seq.outs, ref):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), r
    # new input contents: the replay reads them
    for x in inputs:
        x.copy_(to_dev(_bits(rng, tuple(x.shape)), dev))
    g()
    torch.cuda.synchronize()
    fresh = mxq.LinearSequence(layers, inputs)
    want2 = fresh()
    torch.cuda.synchronize()
    for got, want in zip(seq.outs, want2):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
