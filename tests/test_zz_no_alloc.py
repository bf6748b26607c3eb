"""The allocation-free fused entry point (mxq_quant_gemm_fused_noalloc) against mxq_quant_gemm_fused.

Both run the same kernels, so the outputs must be equal bit for bit.  Each case makes two calls in a row,
the second with a smaller input, so that the second runs over the scratch contents the first left behind;
a full-size MXFP4 case (the FLUX single-stream linear2, 37.6 MB of scratch) sits near the array's limit."""

import numpy as np
import pytest

from tests._util import gpu_or_skip, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_or_skip()


def _pair(fmt, M, K, N, seed, dev, packed):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    g = torch.Generator(device=dev).manual_seed(seed)
    a = (torch.randn((M, K), generator=g, device=dev) * 2.0).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    bias = torch.randn((N,), generator=g, device=dev).to(torch.bfloat16)
    qw = mxq.quantize(fmt, w, packed_scales=packed)
    want = mxq.quant_gemm_fused(a, qw, bias)
    got = torch.empty_like(want)
    mxq.quant_gemm_fused_noalloc(a, qw, bias, got)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("fmt,packed,big,small", [
    ("mxfp8", True, (2048, 3072, 1024), (300, 512, 200)),
    ("mxfp4", False, (1536, 2048, 768), (77, 256, 64)),
    ("nvfp4", False, (1024, 1024, 512), (100, 256, 96)),
    ("mxfp6_e2m3", True, (512, 1024, 640), (33, 256, 40)),
])
def test_noalloc_equals_fused_twice(fmt, packed, big, small, dev):
    import torch

    for i, (M, K, N) in enumerate((big, small)):
        log_case("noalloc", fmt, M, K, N, "call", i)
        got, want = _pair(fmt, M, K, N, 11 + i, dev, packed)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (fmt, M, K, N)
        assert np.isfinite(got.float().cpu().numpy()).all()


def test_noalloc_full_size_mxfp4_linear2(dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, K, N = 4608, 15360, 3072
    assert mxq.workspace_bytes("mxfp4", M, K, True) <= mxq.NOALLOC_SCRATCH_BYTES
    log_case("noalloc full", M, K, N)
    got, want = _pair("mxfp4", M, K, N, 5, dev, True)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_noalloc_rejects_too_large(dev):
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, K = 8192, 8192
    assert mxq.workspace_bytes("mxfp8", M, K, True) > mxq.NOALLOC_SCRATCH_BYTES
    a = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    qw = mxq.quantize("mxfp8", torch.zeros((64, K), dtype=torch.bfloat16, device=dev))
    out = torch.full((M, 64), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(mxq.MxqError) as e:
        mxq.quant_gemm_fused_noalloc(a, qw, None, out)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was launched


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_noalloc_in_graph_replays(fmt, dev):
    """The call it exists for: captured in a HIP graph (it allocates nothing, so capture needs no memory pool
    of its own).  Three replays, each after eager library work that reuses the same per-GPU scratch with
    another shape; every replay equals the workspace call bit for bit."""
    import torch

    from microscaling_quantized_diffusion_amd import mxq

    M, K, N = 1024, 2048, 768
    g = torch.Generator(device=dev).manual_seed(21)
    a = (torch.randn((M, K), generator=g, device=dev) * 2.0).to(torch.bfloat16)
    qw = mxq.quantize(fmt, (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16),
                      packed_scales=fmt != "nvfp4")
    want = mxq.quant_gemm_fused(a, qw)
    out = torch.empty_like(want)
    a2 = (torch.randn((300, 1024), generator=g, device=dev)).to(torch.bfloat16)
    qw2 = mxq.quantize(fmt, (torch.randn((200, 1024), generator=g, device=dev) * 0.02).to(torch.bfloat16),
                       packed_scales=fmt != "nvfp4")
    out2 = torch.empty((300, 200), dtype=torch.bfloat16, device=dev)
    graph = mxq.GraphedCall(lambda: mxq.quant_gemm_fused_noalloc(a, qw, None, out))
    for rep in range(3):
        log_case("noalloc graph", fmt, rep)
        out.zero_()
        mxq.quant_gemm_fused_noalloc(a2, qw2, None, out2)  # eager work over the same scratch
        torch.cuda.synchronize()
        graph()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (fmt, rep)
