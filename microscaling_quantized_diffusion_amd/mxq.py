"""Python binding of libmxq (ctypes): argument marshalling only.

Every step of the quantization and GEMM runs in the library's HIP kernels;
torch is used here only to allocate device memory and to name the current
HIP stream.  If the library is not built, every call raises: there is no
fallback implementation.

Names mirror include/mxq.h.  Formats: "mxfp8", "mxfp4", "nvfp4", "mxfp6_e2m3",
"mxfp6_e3m2".  Calls
that quantize to an MX format take ``scale_rule``: "floor" (the OCP rule,
default) or "rceil" (round the shared scale up, MXQ_SCALE_RCEIL).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Callable, List, Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libmxq.so")

FORMATS = {"mxfp8": 1, "mxfp4": 2, "nvfp4": 3, "mxfp6_e2m3": 4, "mxfp6_e3m2": 5}
SCALE_RULES = {"floor": 0, "rceil": 0x100}  # MXQ_SCALE_RCEIL, OR-ed into the format argument
SCALES_PACKED = 0x200  # MXQ_SCALES_PACKED: MX scales in the GEMM's packed layout (32-row groups, stage-major)
BLOCK = {"mxfp8": 32, "mxfp4": 32, "nvfp4": 16, "mxfp6_e2m3": 32, "mxfp6_e3m2": 32}

MXQ_OK = 0
STATUS_NAMES = {
    0: "MXQ_OK",
    1: "MXQ_ERR_NULL",
    2: "MXQ_ERR_FORMAT",
    3: "MXQ_ERR_SHAPE",
    4: "MXQ_ERR_ALIGN",
    5: "MXQ_ERR_WORKSPACE",
    6: "MXQ_ERR_UNSUPPORTED",
    7: "MXQ_ERR_LAUNCH",
    8: "MXQ_ERR_TOO_LARGE",
}

# (name, restype, argtypes) of every exported entry point
_VP, _I64, _SZ, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "mxq_quantize": (_I, [_I, _VP, _I64, _I64, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "mxq_gemm": (_I, [_I, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mxq_quant_gemm_fused": (_I, [_I, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "mxq_quant_gemm_fused_noalloc": (_I, [_I, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mxq_gemm_requant": (_I, [_I, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _I, _I, _VP, _VP, _VP, _I64, _I64,
                              _VP]),
    "mxq_attention_fp8_requant": (_I, [_I64, _I64, _I64, _I64, _VP, _VP, _VP, _I, _VP, _VP, _I64, _I64, _VP, _SZ,
                                       _VP]),
    "mxq_gemm_bf16": (_I, [_I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "mxq_attention_fp8": (_I, [_I64, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "mxq_attention_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "mxq_workspace_bytes": (_SZ, [_I, _I64, _I64, _I]),
    "mxq_should_quantize": (_I, [_I64, _I64, _I64]),
    "mxq_status_string": (ctypes.c_char_p, [_I]),
    "mxq_abi_version": (_I, []),
}

_lib: Optional[ctypes.CDLL] = None


class MxqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({lib().mxq_status_string(status).decode()})")


def lib() -> ctypes.CDLL:
    """Load libmxq.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m microscaling_quantized_diffusion_amd.build`")
        so = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(so, name)
            fn.restype = res
            fn.argtypes = args
        _lib = so
    return _lib


def _check(fn: str, status: int) -> None:
    if status != MXQ_OK:
        raise MxqError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _fmt(fmt: str, scale_rule: str = "floor") -> int:
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    if scale_rule not in SCALE_RULES:
        raise ValueError(f"unknown scale rule {scale_rule!r}")
    return FORMATS[fmt] | SCALE_RULES[scale_rule]


def _require(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


def code_cols(fmt: str, K: int) -> int:
    """Code bytes per row: MXFP8 one per element, MXFP6 a 32-byte slot per 32-element block, FP4 two codes per byte."""
    if fmt == "mxfp8" or fmt.startswith("mxfp6"):
        return K
    return K // 2


@dataclass
class QTensor:
    """A quantized [rows, K] matrix: codes, scales and (NVFP4) the device per-tensor scale."""

    fmt: str
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: Optional[torch.Tensor]
    K: int
    scales_packed: bool = False  # scales [32 * ceil(rows / 32), K / 32] in the packed layout of include/mxq.h

    @property
    def rows(self) -> int:
        return self.codes.shape[0]


def abi_version() -> int:
    return lib().mxq_abi_version()


def should_quantize(M: int, K: int, N: int) -> bool:
    return bool(lib().mxq_should_quantize(M, K, N))


def workspace_bytes(fmt: str, M: int, K: int, fused: bool) -> int:
    return int(lib().mxq_workspace_bytes(_fmt(fmt), M, K, 1 if fused else 0))


def quantize(fmt: str, x: torch.Tensor, out: Optional[QTensor] = None,
             workspace: Optional[torch.Tensor] = None, scale_rule: str = "floor",
             packed_scales: bool = False) -> QTensor:
    """mxq_quantize: bf16 [rows, K] -> QTensor (codes, scales, tensor scale).  `packed_scales` (MX formats)
    writes the scales in the packed layout the GEMM fetches whole cache lines of (e.g. for weights quantized
    once); a given `out` decides by its own `scales_packed`."""
    _require(x, torch.bfloat16, "x")
    rows, K = x.shape
    dev = x.device
    if out is None:
        codes = torch.empty((rows, code_cols(fmt, K)), dtype=torch.uint8, device=dev)
        srows = (rows + 31) // 32 * 32 if packed_scales else rows
        scales = torch.empty((srows, K // BLOCK[fmt]), dtype=torch.uint8, device=dev)
        ts = torch.empty(1, dtype=torch.float32, device=dev) if fmt == "nvfp4" else None
        out = QTensor(fmt, codes, scales, ts, K, packed_scales)
    f = _fmt(fmt, scale_rule) | (SCALES_PACKED if out.scales_packed else 0)
    need = workspace_bytes(fmt, rows, K, False)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mxq_quantize", lib().mxq_quantize(f, _ptr(x), rows, K, _ptr(out.codes), _ptr(out.scales),
                                              _ptr(out.tensor_scale), _ptr(workspace), wsz, _stream(x)))
    return out


def gemm(a: QTensor, w: QTensor, bias: Optional[torch.Tensor] = None,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_gemm: quantized A [M, K] x quantized W [N, K]^T -> bf16 [M, N]."""
    if a.fmt != w.fmt or a.K != w.K:
        raise ValueError("A and W must share format and K")
    if a.scales_packed != w.scales_packed:
        raise ValueError("A and W must share the scale layout (both packed or both row-major)")
    M, N = a.rows, w.rows
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    f = _fmt(a.fmt) | (SCALES_PACKED if a.scales_packed else 0)
    _check("mxq_gemm", lib().mxq_gemm(f, M, N, a.K, _ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale),
                                      _ptr(w.codes), _ptr(w.scales), _ptr(w.tensor_scale), _ptr(bias), _ptr(out),
                                      _stream(out)))
    return out


def quant_gemm_fused(a: torch.Tensor, w: QTensor, bias: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     scale_rule: str = "floor") -> torch.Tensor:
    """mxq_quant_gemm_fused: bf16 A [M, K] quantized on the fly, times quantized W [N, K]^T -> bf16 [M, N]."""
    _require(a, torch.bfloat16, "a")
    M, K = a.shape
    if K != w.K:
        raise ValueError("K mismatch")
    N = w.rows
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    need = workspace_bytes(w.fmt, M, K, True)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    wsz = workspace.numel() * workspace.element_size()
    f = _fmt(w.fmt, scale_rule) | (SCALES_PACKED if w.scales_packed else 0)
    _check("mxq_quant_gemm_fused",
           lib().mxq_quant_gemm_fused(f, M, N, K, _ptr(a), _ptr(w.codes), _ptr(w.scales), _ptr(w.tensor_scale),
                                      _ptr(bias), _ptr(out), _ptr(workspace), wsz, _stream(a)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MXQ_NOALLOC_SCRATCH_BYTES


def quant_gemm_fused_noalloc(a: torch.Tensor, w: QTensor, bias: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None, scale_rule: str = "floor") -> torch.Tensor:
    """mxq_quant_gemm_fused_noalloc: as quant_gemm_fused, with the activation codes in the library's fixed
    per-GPU scratch array instead of a workspace (pass `out` to allocate nothing at all).  Calls that
    overlap on one GPU share that array and race."""
    _require(a, torch.bfloat16, "a")
    M, K = a.shape
    if K != w.K:
        raise ValueError("K mismatch")
    N = w.rows
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    f = _fmt(w.fmt, scale_rule) | (SCALES_PACKED if w.scales_packed else 0)
    _check("mxq_quant_gemm_fused_noalloc",
           lib().mxq_quant_gemm_fused_noalloc(f, M, N, K, _ptr(a), _ptr(w.codes), _ptr(w.scales),
                                              _ptr(w.tensor_scale), _ptr(bias), _ptr(out), _stream(a)))
    return out


ACTS = {"none": 0, "gelu_tanh": 1}


def _row_strides(q: QTensor):
    """Row strides (bytes) of a quantized output; the codes and scales may be column slices of wider
    matrices (views whose rows are contiguous), e.g. one part of a concatenated activation."""
    for t, n in ((q.codes, "codes"), (q.scales, "scales")):
        if t.dtype != torch.uint8 or t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"{n} must be a uint8 [rows, cols] tensor with contiguous rows")
    return q.codes.stride(0), q.scales.stride(0)


def gemm_requant(a: QTensor, w: QTensor, out_fmt: str, bias: Optional[torch.Tensor] = None, act: str = "none",
                 out: Optional[QTensor] = None, out_bf16: Optional[torch.Tensor] = None,
                 scale_rule: str = "floor") -> QTensor:
    """mxq_gemm_requant: quantized A [M, K] x quantized W [N, K]^T -> act(.) as the next layer's quantized
    activation, a QTensor [M, N] in `out_fmt` (MXFP8 / MXFP4).  `out_bf16` (optional) also receives the bf16
    values that were quantized.  `out` may hold column slices of wider code / scale matrices."""
    if a.fmt != w.fmt or a.K != w.K:
        raise ValueError("A and W must share format and K")
    if a.scales_packed or w.scales_packed:
        raise ValueError("mxq_gemm_requant takes row-major scales")
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    M, N = a.rows, w.rows
    dev = a.codes.device
    if out is None:
        out = QTensor(out_fmt, torch.empty((M, code_cols(out_fmt, N)), dtype=torch.uint8, device=dev),
                      torch.empty((M, N // 32), dtype=torch.uint8, device=dev), None, N)
    qld, sld = _row_strides(out)
    _check("mxq_gemm_requant",
           lib().mxq_gemm_requant(_fmt(a.fmt), M, N, a.K, _ptr(a.codes), _ptr(a.scales), _ptr(w.codes),
                                  _ptr(w.scales), _ptr(bias), ACTS[act], _fmt(out_fmt, scale_rule), _ptr(out_bf16),
                                  _ptr(out.codes), _ptr(out.scales), qld, sld, _stream(a.codes)))
    return out


def gemm_bf16(a: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_gemm_bf16: bf16 A [M, K] x bf16 W [N, K]^T -> bf16 [M, N]."""
    _require(a, torch.bfloat16, "a")
    _require(w, torch.bfloat16, "w")
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _check("mxq_gemm_bf16", lib().mxq_gemm_bf16(M, N, K, _ptr(a), _ptr(w), _ptr(bias), _ptr(out), _stream(a)))
    return out


def attention_workspace_bytes(B: int, H: int, S: int, D: int) -> int:
    return int(lib().mxq_attention_workspace_bytes(B, H, S, D))


def attention_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mxq_attention_fp8: block-scaled FP8 attention of bf16 q, k, v [B, H, S, D] -> bf16 [B, H, S, D]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    B, H, S, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = attention_workspace_bytes(B, H, S, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size()
    _check("mxq_attention_fp8", lib().mxq_attention_fp8(B, H, S, D, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                         _ptr(workspace), wsz, _stream(q)))
    return out


def attention_fp8_requant(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out_fmt: str,
                          out: Optional[QTensor] = None, workspace: Optional[torch.Tensor] = None,
                          scale_rule: str = "floor") -> QTensor:
    """mxq_attention_fp8_requant: the attention output of bf16 q, k, v [B, H, S, D] MX-quantized for the next
    layer, token-major with the heads side by side: a QTensor [B * S, H * D] in `out_fmt`.  `out` may hold
    column slices of wider code / scale matrices (e.g. the attention part of a concatenated activation)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    B, H, S, D = q.shape
    if out is None:
        out = QTensor(out_fmt, torch.empty((B * S, code_cols(out_fmt, H * D)), dtype=torch.uint8, device=q.device),
                      torch.empty((B * S, H * D // 32), dtype=torch.uint8, device=q.device), None, H * D)
    qld, sld = _row_strides(out)
    need = attention_workspace_bytes(B, H, S, D)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size()
    _check("mxq_attention_fp8_requant",
           lib().mxq_attention_fp8_requant(B, H, S, D, _ptr(q), _ptr(k), _ptr(v), _fmt(out_fmt, scale_rule),
                                           _ptr(out.codes), _ptr(out.scales), qld, sld, _ptr(workspace), wsz,
                                           _stream(q)))
    return out


@dataclass
class QuantLinear:
    """A linear layer's weight prepared for selective quantization.

    The weight is quantized once (offline, outside any timed region); the bf16
    copy is kept for calls whose shape falls under the min(M, K, N) < 1024 rule.
    """

    fmt: str
    weight_bf16: Optional[torch.Tensor]
    qweight: Optional[QTensor]
    bias: Optional[torch.Tensor] = None

    @classmethod
    def from_weight(cls, fmt: str, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    keep_bf16: bool = True, quantize_weight: bool = True) -> "QuantLinear":
        # MX weights get the packed scale layout wherever K is whole GEMM stages (the faster GEMM path)
        packed = fmt != "nvfp4" and w.shape[1] % (256 if fmt == "mxfp4" else 128) == 0
        qw = quantize(fmt, w, packed_scales=packed) if quantize_weight else None
        return cls(fmt, w if keep_bf16 else None, qw, bias)

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        M, K = x.shape
        N = (self.qweight.rows if self.qweight is not None else self.weight_bf16.shape[0])
        if self.qweight is not None and should_quantize(M, K, N):
            return quant_gemm_fused(x, self.qweight, self.bias, out, workspace)
        if self.weight_bf16 is None:
            raise ValueError("layer falls back to bf16 but holds no bf16 weight")
        return gemm_bf16(x, self.weight_bf16, self.bias, out)


class LinearSequence:
    """A fixed sequence of linears over static input tensors (one DiT block's
    linears, say), with every output and fused-call workspace preallocated, so
    that calling it allocates nothing and it can be captured into one HIP graph.
    Each layer applies the selective rule as QuantLinear does."""

    def __init__(self, layers: List[QuantLinear], inputs: List[torch.Tensor]):
        if len(layers) != len(inputs):
            raise ValueError("one input per layer")
        self.layers, self.inputs = list(layers), list(inputs)
        self.outs: List[torch.Tensor] = []
        self.workspaces: List[Optional[torch.Tensor]] = []
        for lin, x in zip(self.layers, self.inputs):
            M, K = x.shape
            N = lin.qweight.rows if lin.qweight is not None else lin.weight_bf16.shape[0]
            self.outs.append(torch.empty((M, N), dtype=torch.bfloat16, device=x.device))
            quantized = lin.qweight is not None and should_quantize(M, K, N)
            need = workspace_bytes(lin.fmt, M, K, True) if quantized else 0
            self.workspaces.append(torch.empty(max(need, 1), dtype=torch.uint8, device=x.device) if quantized else None)

    def __call__(self) -> List[torch.Tensor]:
        for lin, x, out, ws in zip(self.layers, self.inputs, self.outs, self.workspaces):
            lin(x, out, ws)
        return self.outs


class GraphedCall:
    """Captures `fn` (library calls on static tensors, issued on torch's current
    stream) into one HIP graph and replays it with a single launch.  `fn` runs
    `warmup` times on a side stream of default priority before capture; the
    library itself allocates, synchronises and memsets nothing, so every entry
    point can be captured.  Replays read the static inputs' current contents."""

    def __init__(self, fn: Callable[[], object], warmup: int = 1):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()

    def __call__(self) -> None:
        self.graph.replay()
