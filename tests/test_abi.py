"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects invalid arguments on the host before anything is launched."""

import ctypes
import os
import re

import pytest

from tests._util import ROOT, ensure_built
from microscaling_quantized_diffusion_amd import mxq

HEADER = os.path.join(ROOT, "include", "mxq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(mxq.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert mxq.abi_version() == 9
    for s in range(9):
        assert lib.mxq_status_string(s)
    assert b"unknown" in lib.mxq_status_string(99)


def test_should_quantize(lib):
    assert mxq.should_quantize(1024, 1024, 1024)
    assert not mxq.should_quantize(1, 3072, 18432)
    assert not mxq.should_quantize(4608, 3072, 1023)
    assert mxq.should_quantize(4608, 15360, 3072)


def test_workspace_sizes(lib):
    assert mxq.workspace_bytes("mxfp8", 4608, 3072, False) == 0
    fused = mxq.workspace_bytes("mxfp8", 4608, 3072, True)
    assert fused >= 4608 * 3072 + 4608 * 96
    assert mxq.workspace_bytes("mxfp4", 4608, 3072, True) >= 4608 * 1536 + 4608 * 96
    assert mxq.workspace_bytes("nvfp4", 16896, 3072, True) >= 16896 * 1536 + 16896 * 192 + 4
    assert mxq.workspace_bytes("nvfp4", 64, 64, False) > 0
    assert lib.mxq_workspace_bytes(9, 16, 32, 1) == 0
    assert lib.mxq_workspace_bytes(1, 16, 33, 1) == 0


P = 4096  # a fake, 16-byte-aligned device address; never dereferenced by these calls


def test_quantize_argument_errors(lib):
    q = lib.mxq_quantize
    assert q(7, P, 4, 32, P, P, None, None, 0, None) == 2  # format
    assert q(1, P, -1, 32, P, P, None, None, 0, None) == 3  # negative rows
    assert q(1, P, 4, 33, P, P, None, None, 0, None) == 3  # K not a multiple of 32
    assert q(3, P, 4, 24, P, P, P, P, 1 << 20, None) == 3  # NVFP4 K not a multiple of 16
    assert q(1, P, 4, 0, P, P, None, None, 0, None) == 3  # K = 0
    assert q(1, None, 4, 32, P, P, None, None, 0, None) == 1  # null input
    assert q(1, P, 4, 32, P, None, None, None, 0, None) == 1  # null scales
    assert q(3, P, 4, 32, P, P, None, P, 1 << 20, None) == 1  # NVFP4 needs the tensor scale
    assert q(1, P + 2, 4, 32, P, P, None, None, 0, None) == 4  # misaligned input
    assert q(3, P, 4, 32, P, P, P, None, 0, None) == 5  # NVFP4 needs a workspace
    assert q(3, P, 4, 32, P, P, P, P, 8, None) == 5  # too small
    assert q(1, P, 0, 32, P, P, None, None, 0, None) == 0  # empty: no-op


def test_gemm_argument_errors(lib):
    g = lib.mxq_gemm
    assert g(0, 4, 4, 32, P, P, None, P, P, None, None, P, None) == 2
    assert g(1, 4, -4, 32, P, P, None, P, P, None, None, P, None) == 3
    assert g(2, 4, 4, 48, P, P, None, P, P, None, None, P, None) == 3
    assert g(1, 4, 4, 32, None, P, None, P, P, None, None, P, None) == 1
    assert g(3, 4, 4, 32, P, P, None, P, P, P, None, P, None) == 1
    assert g(1, 4, 4, 32, P, P, None, P, P, None, None, P + 8, None) == 4
    assert g(1, 0, 4, 32, P, P, None, P, P, None, None, P, None) == 0
    assert g(1, 4, 0, 32, P, P, None, P, P, None, None, P, None) == 0
    assert g(4, 4, 4, 192, P, P, None, P, P, None, None, P, None) == 6  # MXFP6 K not a multiple of 128
    assert g(5, 4, 4, 128, P, P + 1, None, P, P, None, None, P, None) == 4  # MXFP6 scales not 4-byte aligned
    assert lib.mxq_workspace_bytes(4, 64, 256, 1) >= 64 * 256 + 64 * 8  # MXFP6 codes: one byte per element


def test_fused_argument_errors(lib):
    f = lib.mxq_quant_gemm_fused
    need = lib.mxq_workspace_bytes(1, 64, 64, 1)
    assert f(1, 64, 64, 64, P, P, P, None, None, P, None, need, None) == 5
    assert f(1, 64, 64, 64, P, P, P, None, None, P, P, need - 1, None) == 5
    assert f(1, 64, 64, 64, P, P, P, None, None, P, P + 4, need, None) == 4
    assert f(3, 64, 64, 64, P, P, P, None, None, P, P, 1 << 20, None) == 1
    assert f(1, 0, 64, 64, P, P, P, None, None, P, P, need, None) == 0


def test_fused_noalloc_argument_errors(lib):
    """The allocation-free fused call checks its arguments as the fused call does, and rejects a problem
    beyond the fixed scratch array before touching the device."""
    f = lib.mxq_quant_gemm_fused_noalloc
    assert f(9, 64, 64, 64, P, P, P, None, None, P, None) == 2
    assert f(1, 64, 64, 48, P, P, P, None, None, P, None) == 3
    assert f(1, 64, 64, 64, None, P, P, None, None, P, None) == 1
    assert f(1, 64, 64, 64, P, P, P, None, None, P + 2, None) == 4
    assert f(3, 64, 64, 64, P, P, P, None, None, P, None) == 1  # NVFP4 needs W's tensor scale
    assert f(1, 0, 64, 64, P, P, P, None, None, P, None) == 0  # empty: no-op
    big = lib.mxq_workspace_bytes(1, 8192, 8192, 1)
    assert big > mxq.NOALLOC_SCRATCH_BYTES
    assert f(1, 8192, 64, 8192, P, P, P, None, None, P, None) == 8
    assert b"scratch" in lib.mxq_status_string(8)


def test_bf16_argument_errors(lib):
    b = lib.mxq_gemm_bf16
    assert b(4, 4, 0, P, P, None, P, None) == 3
    assert b(4, 4, 8, None, P, None, P, None) == 1
    assert b(4, 4, 8, P, P + 1, None, P, None) == 4
    assert b(0, 4, 8, P, P, None, P, None) == 0


def test_gemm_size_limits(lib):
    """GEMMs beyond K = 2^22 or M * N = 2^39 are rejected before any launch (the
    tile's rows of codes must stay within one 32-bit buffer range)."""
    g, f, b = lib.mxq_gemm, lib.mxq_quant_gemm_fused, lib.mxq_gemm_bf16
    big_k = (1 << 22) + 32
    assert g(1, 4, 4, big_k, P, P, None, P, P, None, None, P, None) == 3
    assert g(3, 4, 4, big_k, P, P, P, P, P, P, None, P, None) == 3
    assert g(1, 1 << 20, (1 << 19) + 1, 32, P, P, None, P, P, None, None, P, None) == 3
    assert f(1, 4, 4, big_k, P, P, P, None, None, P, P, 1 << 40, None) == 3
    assert b(4, 4, (1 << 22) + 1, P, P, None, P, None) == 3
    assert b(1 << 20, (1 << 19) + 1, 8, P, P, None, P, None) == 3
    # the limits themselves are valid shapes: the call proceeds to the pointer checks
    assert g(1, 1 << 20, 1 << 19, 1 << 22, None, P, None, P, P, None, None, P, None) == 1
    assert b(1 << 20, 1 << 19, 1 << 22, None, P, None, P, None) == 1


def test_requant_argument_errors(lib):
    r = lib.mxq_gemm_requant
    # fmt, M, N, K, a_codes, a_scales, w_codes, w_scales, bias, act, out_fmt, out_bf16, out_codes, out_scales,
    # out_codes_ld, out_scales_ld, stream
    assert r(9, 4, 64, 128, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 2  # format
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 7, None, P, P, 0, 0, None) == 2  # output format
    assert r(1, 4, 48, 128, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 3  # N not whole 32-column blocks
    assert r(1, 0, 64, 128, None, None, None, None, None, 0, 1, None, None, None, 0, 0, None) == 0  # empty
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 1, None, None, P, 0, 0, None) == 1  # null codes
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 1, P + 2, P, P, 0, 0, None) == 4  # misaligned bf16 copy
    assert r(1, 4, 64, 96, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 6  # K not a multiple of 128 (FP8)
    assert r(2, 4, 64, 128, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 6  # K not a multiple of 256 (FP4)
    assert r(3, 4, 64, 128, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 6  # NVFP4 operands
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 3, None, P, P, 0, 0, None) == 6  # NVFP4 output
    assert r(1, 4, 64, 128, P, P, P, P, None, 5, 1, None, P, P, 0, 0, None) == 6  # unknown activation
    assert r(4, 4, 64, 192, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 6  # K not a multiple of 128 (FP6)
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 4, None, P, P, 0, 0, None) == 6  # MXFP6 output


RCEIL = 0x100  # MXQ_SCALE_RCEIL


def test_scale_rule_flag(lib):
    """The round-up scale-rule flag is accepted with MX formats wherever a format is taken, and rejected
    with NVFP4 or next to unknown bits, before any pointer is looked at."""
    q, g, f, r = lib.mxq_quantize, lib.mxq_gemm, lib.mxq_quant_gemm_fused, lib.mxq_gemm_requant
    assert q(1 | RCEIL, P, 0, 32, P, P, None, None, 0, None) == 0  # empty: accepted format, no-op
    assert q(2 | RCEIL, None, 4, 32, P, P, None, None, 0, None) == 1  # passes the format check
    assert q(3 | RCEIL, P, 4, 32, P, P, P, P, 1 << 20, None) == 2  # NVFP4 has no such rule
    assert q(1 | 0x400, P, 4, 32, P, P, None, None, 0, None) == 2  # unknown flag bit
    assert q(RCEIL, P, 4, 32, P, P, None, None, 0, None) == 2  # flag without a format
    assert g(1 | RCEIL, 4, 4, 32, None, P, None, P, P, None, None, P, None) == 1  # accepted and ignored
    assert f(2 | RCEIL, 64, 64, 64, P, P, P, None, None, P, None, 0, None) == 5  # passes to the workspace check
    assert f(3 | RCEIL, 64, 64, 64, P, P, P, None, None, P, P, 1 << 20, None) == 2
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 2 | RCEIL, None, None, P, 0, 0, None) == 1  # output rule accepted
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 3 | RCEIL, None, P, P, 0, 0, None) == 2
    assert lib.mxq_workspace_bytes(1 | RCEIL, 64, 64, 1) == lib.mxq_workspace_bytes(1, 64, 64, 1)
    assert lib.mxq_workspace_bytes(3 | RCEIL, 64, 64, 1) == 0
    with pytest.raises(ValueError):
        mxq._fmt("mxfp8", "ceil")


def test_attention_argument_errors(lib):
    a, wb = lib.mxq_attention_fp8, lib.mxq_attention_workspace_bytes
    need = wb(1, 2, 256, 128)
    assert need >= 3 * 2 * 256 * 128
    assert wb(1, 2, 256, 64) == 0 and wb(1, 2, 96, 128) == 0 and wb(-1, 2, 256, 128) == 0
    # B, H, S, D, q, k, v, out, workspace, bytes, stream
    assert a(1, 2, -64, 128, P, P, P, P, P, need, None) == 3  # negative size
    assert a(1, 70000, 64, 128, P, P, P, P, P, need, None) == 3  # B * H beyond one grid dimension
    assert a(0, 2, 256, 128, None, None, None, None, None, 0, None) == 0  # empty
    assert a(1, 2, 256, 64, P, P, P, P, P, need, None) == 6  # head dimension other than 128
    assert a(1, 2, 96, 128, P, P, P, P, P, need, None) == 6  # S not a multiple of 64
    assert a(1, 2, 256, 128, P, None, P, P, P, need, None) == 1
    assert a(1, 2, 256, 128, P, P, P, P + 8, P, need, None) == 4
    assert a(1, 2, 256, 128, P, P, P, P, P, need - 1, None) == 5
    assert a(1, 2, 256, 128, P, P, P, P, None, need, None) == 5


def test_requant_output_strides(lib):
    r, ar = lib.mxq_gemm_requant, lib.mxq_attention_fp8_requant
    # fmt, M, N, K, a_codes, a_scales, w_codes, w_scales, bias, act, out_fmt, out_bf16, out_codes, out_scales,
    # out_codes_ld, out_scales_ld, stream
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 1, None, P, P, 48, 0, None) == 3  # code rows shorter than N
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 2, None, P, P, 0, 1, None) == 3  # scale rows shorter than N/32
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 1, None, P, P, 72, 0, None) == 4  # code stride not 16-aligned
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 1, None, None, P, 128, 8, None) == 1  # valid strides
    need = lib.mxq_attention_workspace_bytes(1, 2, 256, 128)
    # B, H, S, D, q, k, v, out_fmt, out_codes, out_scales, codes_ld, scales_ld, workspace, bytes, stream
    assert ar(1, 2, 256, 128, P, P, P, 3, P, P, 0, 0, P, need, None) == 6  # NVFP4 output
    assert ar(1, 2, 256, 128, P, P, P, 9, P, P, 0, 0, P, need, None) == 2
    assert ar(1, 2, 256, 128, P, P, P, 2, P, P, 64, 0, P, need, None) == 3  # FP4 rows of 128 bytes
    assert ar(1, 2, 256, 128, P, P, P, 1, P, P, 264, 0, P, need, None) == 4
    assert ar(1, 2, 256, 128, P, P, P, 1, None, P, 0, 0, P, need, None) == 1
    assert ar(1, 2, 256, 128, P, P, P, 1, P, P, 0, 0, P, need - 1, None) == 5
    assert ar(0, 2, 256, 128, None, None, None, 1, None, None, 0, 0, None, 0, None) == 0


PACKED = 0x200  # MXQ_SCALES_PACKED


def test_packed_scale_flag(lib):
    """The packed scale layout flag: MX formats with whole GEMM stages only, rejected where it has no
    meaning; every case returns before anything is launched."""
    q, g, f, r = lib.mxq_quantize, lib.mxq_gemm, lib.mxq_quant_gemm_fused, lib.mxq_gemm_requant
    assert q(3 | PACKED, P, 4, 128, P, P, P, P, 1 << 20, None) == 2  # NVFP4
    assert q(1 | PACKED, P, 4, 96, P, P, None, None, 0, None) == 6  # K not whole 128-element stages (FP8)
    assert q(2 | PACKED, P, 4, 128, P, P, None, None, 0, None) == 6  # K not whole 256-element stages (FP4)
    assert q(1 | PACKED, P, 0, 128, P, P, None, None, 0, None) == 0  # empty
    assert g(1 | PACKED, 4, 4, 192, P, P, None, P, P, None, None, P, None) == 6  # K % 128 != 0
    assert g(1 | PACKED, 4, 4, 128, P, P + 1, None, P, P, None, None, P, None) == 4  # scales not 4-byte aligned
    need = lib.mxq_workspace_bytes(1, 64, 128, 1)
    assert lib.mxq_workspace_bytes(1 | PACKED, 64, 128, 1) == need
    assert lib.mxq_workspace_bytes(1, 33, 128, 1) == 4352 + 256  # codes 33 x 128 (to 256 B), scales 64 x 4
    assert f(1 | PACKED, 4, 64, 96, P, P, P, None, None, P, P, need, None) == 6  # K % 128 != 0
    assert f(1 | PACKED, 4, 64, 128, P, P, P + 2, None, None, P, P, need, None) == 4  # W scales not aligned
    assert r(1 | PACKED, 4, 64, 128, P, P, P, P, None, 0, 1, None, P, P, 0, 0, None) == 2  # not for requant
    assert r(1, 4, 64, 128, P, P, P, P, None, 0, 1 | PACKED, None, P, P, 0, 0, None) == 2
