// Device building blocks shared by the GEMM translation units: operand
// vector types, a compile-time loop, MFMA operand packing, and the LDS-staged
// epilogues of the 32x32-MFMA kernels (bf16 output, or the output
// MX-quantized for the next layer).  Everything here is internal to libmxq.
#pragma once

#include <utility>

#include "lds_dma.h"
#include "mx_encode.h"
#include "mxq_internal.h"

namespace mxq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so
// that I can feed immediate operands (MFMA scale byte selects).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ v8i as_v8i(const uint4& lo, const uint4& hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// FP4 operands use only the low four dwords.
__device__ __forceinline__ v8i as_v8i_lo(const uint4& lo) {
  const v4i v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// ------------------------------------------------------------------------
// Epilogue shared by the 32x32-MFMA kernels: out = acc * oscale (+ bias)
// rounded to bf16 (nearest even).  The wave's WTM x WTN sub-tile is staged 32
// rows at a time through `region` (its own EPI_BYTES of idle LDS, 16-byte row
// pad) and written back as 16-byte stores covering whole row segments
// (WTN * 2 contiguous bytes per row), so L2 sees full-line writes instead of
// the accumulator layout's scattered 8-byte pieces.  Lane (r32, q) holds, for
// the 32 x 32 tile (i, j), output row 32j + r32 and columns 32i + 8g + 4q + v
// in acc[i][j][4g + v].
// Output activations applied in fp32 before the bf16 rounding.
enum Act { ACT_NONE = 0, ACT_GELU_TANH = 1 };

// GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), the
// activation between a DiT MLP's up- and down-projections (wavespeed.ai FLUX
// article, model overview: the MLP of each transformer block).  Evaluated as
// x / (1 + exp(-2u)), the same function (0.5 (1 + tanh u) = 1 / (1 + e^-2u)),
// with the hardware exp2 and reciprocal: measured within 1.5 fp32 ulp of the
// fp64 function wherever |GELU(x)| >= 0.25, at a fraction of tanhf's cost.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * u));
}

// Four outputs of lane (r32, q) for the 32 x 32 tile (i, j) and column group g
// (columns nw + 32i + 8g + 4q + v): acc * oscale (+ bias), then the
// activation, rounded to bf16 (nearest even, v_cvt_pk_bf16_f32), packed two
// per dword.
template <int ACT, int TI, int TJ>
__device__ __forceinline__ uint2 epi_bf16x4(const v16f (&acc)[TI][TJ], int i, int j, int g, float oscale,
                                          const uint16_t* __restrict__ bias, int N, int nw, int q) {
  float fv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) fv[v] = acc[i][j][4 * g + v] * oscale;
  if (bias) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int nb = nw + 32 * i + 8 * g + 4 * q + v;
      if (nb < N) fv[v] += bf16_to_f32(bias[nb]);
    }
  }
  if constexpr (ACT == ACT_GELU_TANH) {
#pragma unroll
    for (int v = 0; v < 4; ++v) fv[v] = gelu_tanh(fv[v]);
  }
  const bf16x2 p0 = __builtin_convertvector(f32x2{fv[0], fv[1]}, bf16x2);
  const bf16x2 p1 = __builtin_convertvector(f32x2{fv[2], fv[3]}, bf16x2);
  return make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
}

template <int TI, int TJ, int WTM, int WTN, int ACT = ACT_NONE>
__device__ __forceinline__ void store_tile_bf16(const v16f (&acc)[TI][TJ], float oscale, uint8_t* region,
                                                const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
                                                int M, int N, int mw, int nw, int lane) {
  constexpr int EPI_PITCH = WTN * 2 + 16;
  constexpr int CPRO = WTN * 2 / 16;  // 16-byte chunks per sub-tile row
  constexpr int RPI = 64 / CPRO;      // rows per wave-wide read (lanes past RPI * CPRO idle)
  constexpr int NIT = (32 + RPI - 1) / RPI;
  static_assert(CPRO <= 64, "epilogue read shape");
  const int q = lane >> 5, r32 = lane & 31;
  const bool vec16 = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const int cc = lane % CPRO;
  const int n = nw + 8 * cc;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    if (j > 0) {  // the previous pass's reads are done before its rows are overwritten
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(region + r32 * EPI_PITCH + (32 * i + 8 * g + 4 * q) * 2) =
            epi_bf16x4<ACT>(acc, i, j, g, oscale, bias, N, nw, q);
    // the wave reads back what its own lanes wrote
    wait_lgkmcnt0();
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int lr = it * RPI + lane / CPRO;
      if (lr >= 32 || lane >= RPI * CPRO) continue;
      const uint4 val = *reinterpret_cast<const uint4*>(region + lr * EPI_PITCH + 16 * cc);
      const int m = mw + 32 * j + lr;
      if (m >= M) continue;
      uint16_t* dst = out + (size_t)m * N + n;
      if (vec16 && n + 8 <= N) {
        *reinterpret_cast<uint4*>(dst) = val;
      } else {
        const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// Epilogue that emits the next layer's MX-quantized activations instead of
// (or beside) bf16: the outputs are formed and rounded to bf16 exactly as
// store_tile_bf16 does, then each row's 32-column block is encoded with the
// activation quantizer's arithmetic (mx_encode.h), so the codes and scales
// equal those of quantizing the bf16 output.  Lanes r32 and r32 + 32 hold the
// two 16-column halves of a row's block; their maxima meet through one
// v_permlane32_swap.  Codes are staged through `region` and written as whole
// row segments; requires N % 32 == 0 (whole blocks).  OELEM: 1 = E4M3 codes
// [M, N], 2 = E2M1 codes [M, N/2]; scales E8M0 [M, N/32].
template <int TI, int TJ, int WTM, int WTN, int OELEM, int ACT>
__device__ __forceinline__ void store_tile_requant(const v16f (&acc)[TI][TJ], float oscale, uint8_t* region,
                                                   const uint16_t* __restrict__ bias, uint8_t* __restrict__ qcodes,
                                                   uint8_t* __restrict__ qscales, int M, int N, int mw, int nw,
                                                   int lane, int rceil, int64_t qld, int64_t sld) {
  constexpr int CB = OELEM == 1 ? 32 : 16;  // code bytes per row and 32-column block
  constexpr int RB = TI * CB;               // code bytes per row of the wave's segment
  constexpr int PITCH = RB + 16;
  constexpr int CPR = RB / 16;              // 16-byte chunks per row segment
  constexpr int RPI = 64 / CPR;
  constexpr int NIT = (32 + RPI - 1) / RPI;
  constexpr int COLS_PER_CHUNK = 16 * 32 / CB;
  static_assert(TI <= 8 && CPR <= 64, "requant epilogue shape");
  const int q = lane >> 5, r32 = lane & 31;
  const size_t crow = (size_t)qld;  // code bytes between output rows
  const size_t nsb = (size_t)sld;   // scale bytes between output rows
  const int cc = lane % CPR;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    if (j > 0) {
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
    }
    uint64_t sword = 0;  // scale bytes of blocks i = 0 .. TI-1 of this lane's row
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      uint2 v[4];
      uint32_t m = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v[g] = epi_bf16x4<ACT>(acc, i, j, g, oscale, bias, N, nw, q);
        m = max(m, mx_absmax_bits4(v[g].x, v[g].y));
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(m, m, false, false);
      m = max(sw[0], sw[1]);
      const bool nonfinite = m >= 0x7F80u;  // NaN or Inf in the block: NaN scale, zero codes
      const int e = nonfinite ? 0 : mx_shared_exponent<OELEM>(m, rceil);
      sword |= (uint64_t)(nonfinite ? 0xFFu : (uint32_t)(e + 127)) << (8 * i);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (OELEM == 1) {
          const uint32_t c = nonfinite ? 0u : mx_encode_fp8x4(v[g].x, v[g].y, e);
          *reinterpret_cast<uint32_t*>(region + r32 * PITCH + 32 * i + 8 * g + 4 * q) = c;
        } else {
          const uint32_t c = nonfinite ? 0u : mx_encode_fp4x4<0>(0u, v[g].x, v[g].y, e);
          *reinterpret_cast<uint16_t*>(region + r32 * PITCH + 16 * i + 4 * g + 2 * q) = (uint16_t)c;
        }
      }
    }
    const int mrow = mw + 32 * j + r32;
    if (q == 0 && mrow < M) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
        if (nw + 32 * i < N) qscales[(size_t)mrow * nsb + (size_t)(nw / 32 + i)] = (uint8_t)(sword >> (8 * i));
    }
    wait_lgkmcnt0();
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int lr = it * RPI + lane / CPR;
      if (lr >= 32 || lane >= RPI * CPR) continue;
      const int mr = mw + 32 * j + lr;
      if (mr >= M || nw + cc * COLS_PER_CHUNK >= N) continue;  // whole blocks: a chunk is inside or outside N
      const uint4 val = *reinterpret_cast<const uint4*>(region + lr * PITCH + 16 * cc);
      *reinterpret_cast<uint4*>(qcodes + (size_t)mr * crow + (size_t)nw * CB / 32 + 16 * cc) = val;
    }
  }
}

// Compute units of the current device (cached per device).
inline int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// 256 x 320 tiles instead of 256 x 256 when ceil(tiles / CUs) * width is
// smaller (e.g. 4608 x 12288: 864 tiles in 4 rounds vs 702 tiles in 3).
inline bool mx_prefer_wide_tile(int64_t M, int64_t N, int64_t cus) {
  const int64_t tm = (M + 255) / 256;
  const int64_t r256 = (tm * ((N + 255) / 256) + cus - 1) / cus;
  const int64_t r320 = (tm * ((N + 319) / 320) + cus - 1) / cus;
  return r320 * 320 < r256 * 256;
}

// 384 x 192 tiles (the MX main path only) when ceil(tiles / CUs) * tile area,
// taken 5 % larger, is below that of the 256-row tile the rule above picks:
// 4608 x 12288 is 768 tiles of 384 x 192, three full rounds on 256 CUs,
// against 702 tiles of 256 x 320 whose third round leaves 66 CUs idle.  The
// 5 % is what a 384 x 192 tile measured slower per output than a 256 x 320
// one at equal rounds (nine MFMA tiles per wave instead of ten per barrier).
inline bool mx_prefer_tall_tile(int64_t M, int64_t N, int64_t cus) {
  const int64_t tm = (M + 255) / 256;
  const int64_t c256 = (tm * ((N + 255) / 256) + cus - 1) / cus * (256 * 256);
  const int64_t c320 = (tm * ((N + 319) / 320) + cus - 1) / cus * (256 * 320);
  const int64_t c384 = (((M + 383) / 384) * ((N + 191) / 192) + cus - 1) / cus * (384 * 192);
  return c384 * 21 < (c320 < c256 ? c320 : c256) * 20;
}

}  // namespace
}  // namespace mxq
