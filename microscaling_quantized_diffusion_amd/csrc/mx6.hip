// MXFP6 (E2M3 / E3M2 codes, one E8M0 scale per 32 elements) for gfx950: the
// 6-bit formats of the OCP Microscaling Formats v1.0 specification, the family
// the aitrends.kr MXFP8/NVFP4 article names (Glossary "Microscaling Formats",
// "MXFP8"), beside MXFP8 and MXFP4.
//
// Layout: each 32-element block occupies a 32-byte slot, the 24 bytes of its
// little-endian 192-bit code integer (element j at bits 6j .. 6j+5) followed
// by 8 zero bytes, so a row of K elements is K bytes.  Measured on gfx950,
// this is how the scaled 32x32x64 MFMA reads an FP6 operand: lane half q of
// a row holds the 32 K-elements of K-block q in its first six registers,
// element j at bits 6j of the register tuple, and ignores the last two.  A
// lane therefore loads one slot as is, and the MX GEMM's LDS-DMA ring of
// 128-byte slabs stages FP6 rows exactly as it stages FP8 rows (gemm.hip).
//
// mx6_quant_kernel: one lane per 32-element block: the shared exponent from
// the bf16 bit patterns (the MX rule of mx_encode.h), each element encoded
// round-to-nearest-even with saturation by exact fp32 steps (scale by 2^-e,
// binade from the exponent bits, rintf of the scaled value), one 32-byte
// slot out.
#include "mx_encode.h"
#include "mxq_internal.h"

namespace mxq {
namespace {


// E2M3 (ELEM 3) / E3M2 (ELEM 4) code of an fp32 value y (round to nearest
// even, saturating at the largest magnitude; the sign is kept for zero).
template <int ELEM>
__device__ __forceinline__ uint32_t fp6_encode(float y) {
  constexpr int MB = ELEM == 3 ? 3 : 2;     // mantissa bits
  constexpr int EMIN = ELEM == 3 ? 0 : -2;  // 1 - bias: exponent of the smallest normal
  constexpr float MAXV = ELEM == 3 ? 7.5f : 28.0f;
  const uint32_t sign = (__float_as_uint(y) >> 31) << 5;
  const float a = fabsf(y);
  if (a >= MAXV) return sign | 0x1Fu;
  // binade of a (fp32 zeros and subnormals lie far below 2^EMIN)
  const int E = max((int)((__float_as_uint(a) >> 23) & 0xFFu) - 127, EMIN);
  // grid step 2^(E - MB): scaling by a power of two is exact, rintf rounds half to even
  const float qf = rintf(a * __uint_as_float((uint32_t)(MB - E + 127) << 23));
  return sign | (uint32_t)((E - EMIN) * (1 << MB) + (int)qf);
}

template <int ELEM>
__global__ __launch_bounds__(256) void mx6_quant_kernel(const uint4* __restrict__ x, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, int64_t nblocks, int rceil) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += stride) {
    uint32_t w[16];  // 32 bf16, element 2k in the low half of w[k]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 v = x[4 * b + u];
      w[4 * u] = v.x;
      w[4 * u + 1] = v.y;
      w[4 * u + 2] = v.z;
      w[4 * u + 3] = v.w;
    }
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, mx_absmax_bits4(w[2 * k], w[2 * k + 1]));
    uint64_t pk[3] = {0, 0, 0};
    uint32_t sbyte = 0xFFu;  // NaN or Inf in the block: NaN scale, zero codes
    if (m < 0x7F80u) {
      const int e = mx_shared_exponent<ELEM>(m, rceil);
      sbyte = (uint32_t)(e + 127);
      const float inv = mx_pow2f(-e);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t h = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint64_t c = fp6_encode<ELEM>(__uint_as_float(h << 16) * inv);
        constexpr int kBits = 6;
        const int bit = kBits * j;
        pk[bit >> 6] |= c << (bit & 63);
        if ((bit & 63) > 58) pk[(bit >> 6) + 1] |= c >> (64 - (bit & 63));
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
    dst[0] = make_uint4((uint32_t)pk[0], (uint32_t)(pk[0] >> 32), (uint32_t)pk[1], (uint32_t)(pk[1] >> 32));
    dst[1] = make_uint4((uint32_t)pk[2], (uint32_t)(pk[2] >> 32), 0u, 0u);
    scales[b] = (uint8_t)sbyte;
  }
}

int quant_grid(int64_t nblocks) {
  int64_t g = (nblocks + 255) / 256;
  if (g > 8192) g = 8192;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t launch_mx6_quant(int elem, int rceil, const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes,
                            uint8_t* scales, hipStream_t stream) {
  const int64_t nblocks = rows * cols / 32;
  if (nblocks == 0) return hipSuccess;
  const int grid = quant_grid(nblocks);
  if (elem == 3)
    hipLaunchKernelGGL(mx6_quant_kernel<3>, dim3(grid), dim3(256), 0, stream, (const uint4*)x, codes, scales, nblocks,
                       rceil);
  else
    hipLaunchKernelGGL(mx6_quant_kernel<4>, dim3(grid), dim3(256), 0, stream, (const uint4*)x, codes, scales, nblocks,
                       rceil);
  return hipGetLastError();
}

}  // namespace mxq
