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


def row_major_scales(q) -> np.ndarray:
    """A QTensor's scales as a row-major [rows, K/32] numpy array, undoing the packed layout if it has one
    (block kb of row r at (r // 32) * 32 S + (kb // P) * 32 P + (r % 32) * P + kb % P, P = 8 for MXFP4 else 4)."""
    s = q.scales.cpu().numpy()
    if not getattr(q, "scales_packed", False):
        return s
    rows, S = q.rows, q.K // 32
    P = 8 if q.fmt == "mxfp4" else 4
    r = np.arange(rows)[:, None]
    kb = np.arange(S)[None, :]
    return s.reshape(-1)[(r // 32) * 32 * S + (kb // P) * 32 * P + (r % 32) * P + kb % P]
