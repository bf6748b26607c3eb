// MX GEMM with the requantizing epilogue (producer-fused quantization): the
// instantiations of mxe_gemm_kernel (gemm_mx_kernel.h) whose epilogue applies
// the optional activation and MX-quantizes the output for the next layer,
// on the same tiles as the bf16-output GEMM (256 x 320 only for FP8 / FP6
// operands; FP4 operands take 256 x 256 there).
#include "gemm_mx_kernel.h"

namespace mxq {
namespace {

struct ReqArgs {
  int64_t M, N, K;
  const uint8_t *a, *as, *w, *ws;
  const uint16_t* bias;
  uint16_t* out;
  uint8_t *qcodes, *qscales;
  int rceil;
  int64_t qld, sld;
  hipStream_t stream;
};

template <int ELEM, int OELEM, int ACT, int BN, int D, int E, int BM = 256>
hipError_t launch_req(const ReqArgs& r) {
  return launch_mxe<ELEM, OELEM, ACT, 0, BN, D, E, BM>(r.M, r.N, r.K, r.a, r.as, r.w, r.ws, r.bias, r.out, r.stream,
                                                       r.qcodes, r.qscales, r.rceil, r.qld, r.sld);
}

template <int ELEM, int OELEM, int ACT>
hipError_t launch_req_tile(MxTile tile, const ReqArgs& r) {
  if (tile == MX_TILE_384x192) return launch_req<ELEM, OELEM, ACT, 192, 1, 3, 384>(r);
  if constexpr (ELEM != 2) {
    if (tile == MX_TILE_256x320) return launch_req<ELEM, OELEM, ACT, 320, 1, 6>(r);
  }
  return launch_req<ELEM, OELEM, ACT, 256, 2, 2>(r);
}

template <int ELEM>
hipError_t launch_req_elem(int out_elem, int act, MxTile tile, const ReqArgs& r) {
  if (out_elem == 1)
    return act == ACT_GELU_TANH ? launch_req_tile<ELEM, 1, ACT_GELU_TANH>(tile, r)
                                : launch_req_tile<ELEM, 1, ACT_NONE>(tile, r);
  return act == ACT_GELU_TANH ? launch_req_tile<ELEM, 2, ACT_GELU_TANH>(tile, r)
                              : launch_req_tile<ELEM, 2, ACT_NONE>(tile, r);
}

}  // namespace

hipError_t launch_mx_staged_requant(int elem, int out_elem, int out_rceil, int act, MxTile tile, int64_t M, int64_t N,
                                    int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                                    const uint8_t* w_codes, const uint8_t* w_scales, const uint16_t* bias,
                                    uint16_t* out_bf16, uint8_t* out_codes, uint8_t* out_scales, int64_t qld,
                                    int64_t sld, hipStream_t stream) {
  const ReqArgs r{M, N, K, a_codes, a_scales, w_codes, w_scales, bias, out_bf16, out_codes, out_scales, out_rceil,
                  qld, sld, stream};
  switch (elem) {
    case 1: return launch_req_elem<1>(out_elem, act, tile, r);
    case 2: return launch_req_elem<2>(out_elem, act, tile, r);
    case 3: return launch_req_elem<3>(out_elem, act, tile, r);
    case 4: return launch_req_elem<4>(out_elem, act, tile, r);
  }
  return hipErrorInvalidValue;
}

}  // namespace mxq
