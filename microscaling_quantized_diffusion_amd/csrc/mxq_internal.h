// Internal declarations shared by the HIP translation units of libmxq.
// Nothing here is part of the public ABI (include/mxq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxq.h"

namespace mxq {

// ---------------------------------------------------------------- launchers
// Each launcher enqueues its kernels on `stream` and returns the HIP error of
// the launch (hipSuccess when nothing failed).  Shapes are already validated.

// MX quantizer: x bf16 [rows, cols] -> codes / E8M0 scales.  elem: 1 = E4M3,
// 2 = E2M1, 3 = E2M3, 4 = E3M2 (FP6 codes: a 32-byte slot per 32-element
// block, element j at bits 6j of the slot's little-endian 192-bit integer,
// then 8 zero bytes); rceil: 0 = floor shared-exponent rule, 1 = round-up
// rule; packed: scales in the GEMM's packed layout (32-row groups,
// stage-major; needs rows * cols / 32 < 2^32 and whole stages in cols).
hipError_t launch_mx_quant(int elem, int rceil, int packed, const uint16_t* x, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);

// NVFP4 quantizer (two kernels: global-amax partials, then block quantization).
// `partials` holds nvfp4_partials_count(rows*cols) uint32 values.
int64_t nvfp4_partials_count(int64_t n_elems);
hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              float* tensor_scale, uint32_t* partials, hipStream_t stream);

// MX GEMM (elem: 1 = E4M3, 2 = E2M1, 3 = E2M3, 4 = E3M2; the FP6 formats
// need K % 128 == 0 and 4-byte aligned scale rows, else hipErrorInvalidValue;
// packed: both operands' scales in the packed layout, which needs the same).
hipError_t launch_mx_gemm(int elem, int packed, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                          const uint16_t* bias, uint16_t* out, hipStream_t stream);

// Output tile of the early-published MX main-path GEMM.
enum MxTile { MX_TILE_256x256 = 0, MX_TILE_256x320 = 1, MX_TILE_384x192 = 2 };
// The early-published MX main-path GEMM (gemm_mx.hip): whole stages
// (K % 128 == 0, FP4 K % 256 == 0) and 4-byte aligned scale rows, for the
// formats and tiles where mx_staged_supports(elem, tile) holds.
bool mx_staged_supports(int elem, MxTile tile);
hipError_t launch_mx_staged(int elem, int packed, MxTile tile, int64_t M, int64_t N, int64_t K,
                            const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                            const uint8_t* w_scales, const uint16_t* bias, uint16_t* out, hipStream_t stream);
// The same kernel with the requantizing epilogue (gemm_mx_requant.hip), as
// launch_mx_gemm_requant describes it; tile 256 x 320 needs elem != 2.
hipError_t launch_mx_staged_requant(int elem, int out_elem, int out_rceil, int act, MxTile tile, int64_t M, int64_t N,
                                    int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                                    const uint8_t* w_codes, const uint8_t* w_scales, const uint16_t* bias,
                                    uint16_t* out_bf16, uint8_t* out_codes, uint8_t* out_scales, int64_t qld,
                                    int64_t sld, hipStream_t stream);

// MX GEMM whose epilogue emits the output MX-quantized (out_elem: 1 = E4M3,
// 2 = E2M1; E8M0 scales per 32 output columns, shared-exponent rule as in
// launch_mx_quant), after an optional activation (act: 0 none, 1 GELU tanh
// form); out_bf16 (nullable) also receives the bf16 values that were
// quantized.  codes_ld / scales_ld: bytes between output rows of the codes
// and scales (0 = dense, N or N/2 and N/32).  Only where
// mx_requant_supported() holds.
bool mx_requant_supported(int elem, int64_t N, int64_t K, const uint8_t* a_scales, const uint8_t* w_scales);
hipError_t launch_mx_gemm_requant(int elem, int out_elem, int out_rceil, int act, int64_t M, int64_t N, int64_t K,
                                  const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                                  const uint8_t* w_scales, const uint16_t* bias, uint16_t* out_bf16,
                                  uint8_t* out_codes, uint8_t* out_scales, int64_t codes_ld, int64_t scales_ld,
                                  hipStream_t stream);

// NVFP4 GEMM.
hipError_t launch_nvfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_ts, const uint8_t* w_codes, const uint8_t* w_scales,
                             const float* w_ts, const uint16_t* bias, uint16_t* out, hipStream_t stream);

// Block-scaled FP8 attention, head dimension 128, S a multiple of 64.  The
// workspace holds the MXFP8 Q and K (codes [BH*S, 128], scales [BH*S, 4]) and
// V^T (codes [BH*128, S]; scales tile-major [BH][S/64][128][2], one 256-byte
// run per 64-key tile), each section 256-byte aligned; q, k, v, out are bf16
// [BH, S, 128].
struct AttentionLayout {
  size_t q_codes, q_scales, k_codes, k_scales, vt_codes, vt_scales, total;
};
// out_elem 0: bf16 output `out` [BH, S, 128].  out_elem 1 / 2: the same
// values MX-quantized (E4M3 / E2M1, rceil selecting the scale rule) into
// qcodes / qscales token-major: row b*S + s, columns h*128 + d (H heads per
// batch), rows qld and sld bytes apart.
AttentionLayout attention_layout(int64_t BH, int64_t S);
hipError_t launch_attention_fp8(int64_t BH, int64_t S, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* out, uint8_t* workspace, hipStream_t stream, int out_elem = 0,
                                int rceil = 0, int64_t H = 1, uint8_t* qcodes = nullptr, uint8_t* qscales = nullptr,
                                int64_t qld = 0, int64_t sld = 0);

// bf16 GEMM.
hipError_t launch_bf16_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* a, const uint16_t* w,
                            const uint16_t* bias, uint16_t* out, hipStream_t stream);

// ------------------------------------------------------------ device helpers

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Remap a linear workgroup id so that each of the 8 XCDs (which receive
// workgroups round-robin) works on one contiguous range of ids.
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t id, uint32_t n) {
  const uint32_t xcds = 8;
  uint32_t per = n / xcds;  // ids [0, per*xcds) are remapped; the tail keeps its id
  if (id >= per * xcds) return id;
  return (id % xcds) * per + id / xcds;
}

}  // namespace mxq
