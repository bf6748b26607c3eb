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


def oracle_rows(fn, bits: np.ndarray, *args, workers: int = 16, chunk: int = 1024):
    """Apply a row-wise oracle quantizer (MX, or NVFP4 with its tensor scale given) to row chunks of `bits`
    in a thread pool and concatenate the per-row outputs.  Rows are quantized independently, so the result
    equals fn(bits, *args); NumPy releases the GIL inside the large array operations, which makes the
    oracle affordable on full-size tensors.  The oracle itself is unchanged."""
    from concurrent.futures import ThreadPoolExecutor

    parts = [np.ascontiguousarray(bits[r:r + chunk]) for r in range(0, bits.shape[0], chunk)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(lambda p: fn(p, *args), parts))
    out = [np.concatenate([r[i] for r in res]) for i in range(2)]
    return tuple(out) + tuple(res[0][2:])


def fused_workspace_a(fmt: str, M: int, K: int, ws, packed: bool):
    """The activation codes [M, code bytes] and row-major scales [M, K/block] that mxq_quant_gemm_fused left
    in its workspace.  The workspace layout is the library's own: codes at byte 0, then the scales at the next
    256-byte boundary (MX scales in the packed layout when the weights' scales are packed, with rows padded
    to whole groups of 32); a change there fails these tests loudly."""
    cb = M * (K if fmt == "mxfp8" or fmt.startswith("mxfp6") else K // 2)
    s0 = (cb + 255) // 256 * 256
    blk = 16 if fmt == "nvfp4" else 32
    S = K // blk
    w = ws.cpu().numpy()
    codes = w[:cb].reshape(M, -1)
    if not packed:
        return codes, w[s0:s0 + M * S].reshape(M, S)
    P = 8 if fmt == "mxfp4" else 4
    rows = (M + 31) // 32 * 32
    flat = w[s0:s0 + rows * S]
    r = np.arange(M)[:, None]
    kb = np.arange(S)[None, :]
    return codes, flat[(r // 32) * 32 * S + (kb // P) * 32 * P + (r % 32) * P + kb % P]
