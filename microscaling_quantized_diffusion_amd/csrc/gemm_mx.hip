// MX block-scaled GEMM main path with a bf16 output: the tile choice and the
// instantiations of mxe_gemm_kernel (gemm_mx_kernel.h) for every MX format.
#include "gemm_mx_kernel.h"

namespace mxq {
namespace {

// 256 x 256 tiles with a two-group read lookahead and the DMA spread over
// two head groups; 256 x 320 tiles (160 accumulators per wave) with a
// one-group lookahead, which is what fits the registers without spilling
// (FP8 and FP6 only: FP4 at 320 columns spills), and six head groups;
// 384 x 192 tiles (144 accumulators, three MFMA tiles each way per wave) with
// a one-group lookahead and three head groups (E = 3 measured 1-2 % faster
// than E = 2 or 4 on the FLUX shapes).
template <int ELEM, int PK>
hipError_t launch_mxe_tile(MxTile tile, int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                           const uint8_t* w, const uint8_t* ws, const uint16_t* bias, uint16_t* out,
                           hipStream_t stream) {
  if (tile == MX_TILE_384x192)
    return launch_mxe<ELEM, 0, ACT_NONE, PK, 192, 1, 3, 384>(M, N, K, a, as, w, ws, bias, out, stream, nullptr, nullptr,
                                                             0, 0, 0);
  if constexpr (ELEM != 2) {
    if (tile == MX_TILE_256x320)
      return launch_mxe<ELEM, 0, ACT_NONE, PK, 320, 1, 6>(M, N, K, a, as, w, ws, bias, out, stream, nullptr, nullptr, 0, 0,
                                                          0);
  }
  return launch_mxe<ELEM, 0, ACT_NONE, PK, 256, 2, 2>(M, N, K, a, as, w, ws, bias, out, stream, nullptr, nullptr, 0, 0,
                                                      0);
}

template <int PK>
hipError_t launch_mxe_elem(int elem, MxTile tile, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                           const uint8_t* as, const uint8_t* w, const uint8_t* ws, const uint16_t* bias,
                           uint16_t* out, hipStream_t stream) {
  switch (elem) {
    case 1: return launch_mxe_tile<1, PK>(tile, M, N, K, a, as, w, ws, bias, out, stream);
    case 2: return launch_mxe_tile<2, PK>(tile, M, N, K, a, as, w, ws, bias, out, stream);
    case 3: return launch_mxe_tile<3, PK>(tile, M, N, K, a, as, w, ws, bias, out, stream);
    case 4: return launch_mxe_tile<4, PK>(tile, M, N, K, a, as, w, ws, bias, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool mx_staged_supports(int elem, MxTile tile) { return !(tile == MX_TILE_256x320 && elem == 2); }

hipError_t launch_mx_staged(int elem, int packed, MxTile tile, int64_t M, int64_t N, int64_t K,
                            const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                            const uint8_t* w_scales, const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  return packed ? launch_mxe_elem<1>(elem, tile, M, N, K, a_codes, a_scales, w_codes, w_scales, bias, out, stream)
                : launch_mxe_elem<0>(elem, tile, M, N, K, a_codes, a_scales, w_codes, w_scales, bias, out, stream);
}

}  // namespace mxq
