"""Microscaling-quantized GEMM for diffusion-transformer linears on MI355X (gfx950).

Dynamic block-scaled quantization of bf16 activations (MXFP8, MXFP4, NVFP4-style)
fused with a block-scaled GEMM against pre-quantized weights, with a bf16
fallback for layers whose smallest dimension is below 1024.  The compute runs
in hand-written HIP kernels behind the C ABI of ``include/mxq.h``
(``libmxq.so``); ``mxq`` is its Python binding and ``inputs`` draws the seeded
synthetic FLUX-shaped workloads.
"""

__all__ = ["mxq", "inputs", "build"]
