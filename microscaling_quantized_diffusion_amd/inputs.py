"""Seeded synthetic inputs shaped like FLUX DiT linear layers.

This module only draws random numbers and rounds them to bf16; it holds none
of the quantization or GEMM arithmetic, so both the HIP path (through the
tests and the benchmark) and the CPU oracle can consume the same inputs.

Shapes stand in for the FLUX-dev transformer linears of the diffusion
workloads the pages discuss (wavespeed.ai FLUX-dev on B200, "FLUX-Dev";
aitrends.kr MXFP8/NVFP4 article, "Section details"; devin.kr TensorRT-LLM
VisualGen article at 2048x2048): hidden size 3072, MLP width 12288,
1024x1024 images giving 4096 image tokens plus 512 text tokens (M = 4608)
and 2048x2048 giving 16384 + 512 (M = 16896).  No trained weights or
prompts are used: activations and weights are synthetic.

Distributions ("N(mu, s)" means standard deviation s):
  rowscale  : N(0, 1) times a per-row factor exp(N(0, 0.5))
  outlier   : N(0, 1) with round(0.01 * K) input channels (columns)
              chosen without replacement and multiplied by 20
  student_t : Student-t with 4 degrees of freedom, unit scale
  weights   : N(0, 0.02)
Draw order within one case: activation base, row factors, outlier channel
indices, weights; every case is seeded (seed 0 by default) with numpy's
PCG64 ``default_rng``.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def gen_activation(rng: np.random.Generator, M: int, K: int, kind: str) -> np.ndarray:
    """bf16 bit patterns [M, K] drawn from one of the activation distributions."""
    if kind == "rowscale":
        base = rng.standard_normal((M, K), dtype=np.float32)
        rows = np.exp(rng.normal(0.0, 0.5, size=(M, 1))).astype(np.float32)
        x = base * rows
    elif kind == "outlier":
        x = rng.standard_normal((M, K), dtype=np.float32)
        n_out = int(round(0.01 * K))
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(20.0)
    elif kind == "student_t":
        x = rng.standard_t(4, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    return bf16_bits_from_f32(x)


def gen_weight(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """bf16 bit patterns [N, K] ~ N(0, 0.02)."""
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return bf16_bits_from_f32(w)


@dataclass(frozen=True)
class Linear:
    """One linear layer out = A @ W^T with A [M, K] and W [N, K]."""

    name: str
    M: int
    K: int
    N: int
    fmt: str  # "mxfp8" | "mxfp4" | "mxfp6_e2m3" | "mxfp6_e3m2" | "nvfp4" (bf16 when the selective rule says so)
    act: str


@dataclass(frozen=True)
class Workload:
    name: str
    layers: List[Linear] = field(default_factory=list)
    description: str = ""


def _double_block(batch: int) -> Workload:
    M = 4608 * batch
    return Workload(
        f"flux_double_block_b{batch}",
        [
            Linear("qkv", M, 3072, 9216, "mxfp8", "rowscale"),
            Linear("proj", M, 3072, 3072, "mxfp8", "rowscale"),
            Linear("mlp_up", M, 3072, 12288, "mxfp8", "rowscale"),
            Linear("mlp_down", M, 12288, 3072, "mxfp8", "rowscale"),
            Linear("modulation", batch, 3072, 18432, "mxfp8", "rowscale"),
        ],
        f"one FLUX double-stream block's linears at batch {batch}, 1024x1024 (M = 4608*{batch}); "
        "the modulation linear (M = batch) falls back to bf16 by the min(M,K,N) < 1024 rule",
    )


WORKLOADS: Dict[str, Workload] = {
    "mxfp8_1024": Workload(
        "mxfp8_1024",
        [Linear("square", 1024, 1024, 1024, "mxfp8", "rowscale")],
        "single MXFP8 quant+GEMM, 1024^3",
    ),
    "flux_mlp_up_mxfp8": Workload(
        "flux_mlp_up_mxfp8",
        [Linear("mlp_up", 4608, 3072, 12288, "mxfp8", "outlier")],
        "FLUX-dev MLP up-projection at 1024x1024 (4096 image + 512 text tokens), MXFP8",
    ),
    "flux_mlp_up_mxfp6": Workload(
        "flux_mlp_up_mxfp6",
        [
            Linear("mlp_up_e2m3", 4608, 3072, 12288, "mxfp6_e2m3", "outlier"),
            Linear("mlp_up_e3m2", 4608, 3072, 12288, "mxfp6_e3m2", "outlier"),
        ],
        "FLUX-dev MLP up-projection at 1024x1024 in the two MXFP6 element formats",
    ),
    "flux_single_mxfp4": Workload(
        "flux_single_mxfp4",
        [
            Linear("linear1", 4608, 3072, 21504, "mxfp4", "rowscale"),
            Linear("linear2", 4608, 15360, 3072, "mxfp4", "rowscale"),
        ],
        "FLUX single-stream block linears in MXFP4",
    ),
    "flux_2048_nvfp4": Workload(
        "flux_2048_nvfp4",
        [Linear("mlp_up", 16896, 3072, 12288, "nvfp4", "student_t")],
        "NVFP4-style GEMM at 2048x2048 (16384 image + 512 text tokens)",
    ),
    "flux_double_block_b1": _double_block(1),
    "flux_double_block_b4": _double_block(4),
}


def make_layer_inputs(layer: Linear, seed: int = 0, M: Optional[int] = None, K: Optional[int] = None,
                      N: Optional[int] = None):
    """(A bits [M,K], W bits [N,K]) for a layer; M/K/N may be overridden to shrink a case."""
    M = layer.M if M is None else M
    K = layer.K if K is None else K
    N = layer.N if N is None else N
    rng = np.random.default_rng(seed)
    a = gen_activation(rng, M, K, layer.act)
    w = gen_weight(rng, N, K)
    return a, w
