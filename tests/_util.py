"""Shared helpers for the GPU parity tests (no quantization arithmetic here)."""

import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_built():
    """Load the in-tree library, building it only when nothing is built."""
    from microscaling_quantized_diffusion_amd import mxq

    if not os.path.exists(mxq.LIB_PATH):
        from microscaling_quantized_diffusion_amd import build

        build.build()
    return mxq.lib()


def gpu_or_skip():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dev):
    """uint16 bf16 bit patterns -> bf16 CUDA tensor (bit-exact)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_np_u8(t):
    return t.cpu().numpy()


def bf16_out_to_f64(t):
    import torch

    return t.float().cpu().numpy().astype(np.float64)


def log_case(*parts):
    print("CASE", *parts, flush=True)
