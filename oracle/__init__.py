"""CPU oracle for block-scaled ("microscaling") quantization and GEMM.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct reference that the HIP path is checked against.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product path (the HIP library and its Python binding) never does,
and the two share no code, tables or helpers.

What it computes, and where the pages define it:

* Microscaling block quantization: a short block of consecutive elements
  shares one high-precision scale factor so that a low-bit element format
  keeps a wide dynamic range.  aitrends.kr "Accelerating diffusion-model
  inference with MXFP8 and NVFP4 quantization on NVIDIA B200", Glossary
  ("Microscaling Formats").
* MXFP8 is the OCP-standard 8-bit microscaling format (same page, Glossary
  "MXFP8"); its element and scale encodings (E4M3, E8M0) and the shared-
  exponent rule are taken from the public OCP Microscaling Formats (MX) v1.0
  specification, which that entry names.  The same specification's 6-bit
  formats (MXFP6: E2M3, E3M2) are offered beside MXFP8 and MXFP4.
* NVFP4 (same page, Glossary "NVFP4"; dynamic per-tensor scale in the
  TorchAO configuration shown under "Section details") is read as E2M1
  elements with one E4M3 scale per 16 elements and one fp32 per-tensor scale
  derived from the global absolute maximum.
* Attention in 8-bit floating point with per-token correction of the
  quantization error (devin.kr article on FLUX image generation accelerated
  on Blackwell, "Compute efficiency and acceleration"); the steps are
  readings, stated in ``attention``.
* Dynamic activation quantization followed by a low-precision GEMM against
  pre-quantized weights (same page, "Section details": the NVFP4 dynamic-
  activation / NVFP4-weight configuration), with layers whose smallest GEMM
  dimension is below 1024 left in bf16 (same page, "Section details",
  second "Evidence" block, selective quantization).

Modules
-------
formats  closed-form decode of bf16 / E4M3 / E2M1 / E8M0 and the
         round-to-nearest-even saturating element encoder (numpy, fp64).
exact    scalar reference in exact rational arithmetic (fractions.Fraction)
         used to pin the vectorized code on small and exhaustive cases.
quant    MXFP8 / MXFP4 / NVFP4 quantizers and dequantizers (numpy, fp64).
gemm     fp64 GEMM references, the normwise error metric and the GELU
         (tanh form) applied before an epilogue's requantization.
attention  block-scaled FP8 attention (MXFP8 Q, K along the head dimension,
         V along tokens, online softmax over key tiles with P in E4M3 at a
         fixed 2^8 scale) and textbook softmax attention, in float64.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, exhaustive brute force, library decoders and hand-
worked fixtures under ``tests/golden/``; none is "parity unpinned".
"""

from .formats import (  # noqa: F401
    E2M1,
    E4M3,
    ElemFormat,
    decode_bf16,
    decode_e4m3,
    decode_e2m1,
    decode_e8m0,
    encode,
)
from .quant import (  # noqa: F401
    MXFP4,
    MXFP6_E2M3,
    MXFP6_E3M2,
    MXFP8,
    NVFP4,
    dequant_mx,
    dequant_nvfp4,
    nvfp4_tensor_scale,
    quantize_mx,
    quantize_nvfp4,
    should_quantize,
    pack_fp6,
    unpack_fp4,
    unpack_fp6,
)
from .gemm import (  # noqa: F401
    bf16_half_ulp,
    bf16_round,
    gelu_tanh,
    gemm_error,
    gemm_error_rows,
    rounding_mismatch_rate,
    gemm_bf16_ref,
    gemm_mx_ref,
    gemm_nvfp4_ref,
    normwise_error,
)
