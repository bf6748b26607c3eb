// MXFP6 (E2M3 / E3M2 codes, one E8M0 scale per 32 elements) for gfx950: the
// 6-bit formats of the OCP Microscaling Formats v1.0 specification, the family
// the aitrends.kr MXFP8/NVFP4 article names (Glossary "Microscaling Formats",
// "MXFP8"), beside MXFP8 and MXFP4.
//
// Layout: each 32-element block is 24 bytes, element j at bits 6j .. 6j+5 of
// the block's little-endian 192-bit integer.  Measured on gfx950, this is how
// the scaled 32x32x64 MFMA reads an FP6 operand: lane half q of a row holds
// the 32 K-elements of K-block q in its first six registers, element j at
// bits 6j of the register tuple, so a lane loads one block's 24 bytes as is.
//
// Kernels
//   mx6_quant_kernel  one lane per 32-element block: the shared exponent from
//                     the bf16 bit patterns (the MX rule of mx_encode.h), each
//                     element encoded round-to-nearest-even with saturation by
//                     exact fp32 steps (scale by 2^-e, binade from the
//                     exponent bits, rintf of the scaled value), 24 bytes out.
//   mx6_gemm_kernel   a 128 x 128 output tile per workgroup, four waves of
//                     64 x 64 (2 x 2 scaled 32x32x64 MFMAs with the FP6
//                     format code); 128 K-elements (96 code bytes per row)
//                     staged in LDS per iteration, the next stage's loads in
//                     flight in registers meanwhile; bf16 epilogue with
//                     optional bias.  A plain design: the MX GEMM's LDS-DMA
//                     ring is built around 16-byte chunks of 128-byte slabs,
//                     which 24-byte blocks do not fit.
#include "mx_encode.h"
#include "mxq_internal.h"

namespace mxq {
namespace {

typedef int m6_v8i __attribute__((ext_vector_type(8)));
typedef float m6_v16f __attribute__((ext_vector_type(16)));
typedef float m6_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 m6_bf16x2 __attribute__((ext_vector_type(2)));

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
    uint64_t* dst = reinterpret_cast<uint64_t*>(codes + 24 * b);
    dst[0] = pk[0];
    dst[1] = pk[1];
    dst[2] = pk[2];
    scales[b] = (uint8_t)sbyte;
  }
}

constexpr int kT = 128;          // output tile rows and columns
constexpr int kStageBlocks = 4;  // 32-element blocks per row and stage (128 K-elements, 2 MFMA steps)
constexpr int kRowB = kStageBlocks * 24;  // 96 code bytes per row and stage
constexpr int kPitch = 104;      // LDS bytes per staged row: 8-byte aligned, 26 dwords (spreads the banks)
constexpr int kChunks = kT * kRowB / 16;  // 16-byte chunks per operand and stage (768, 3 per thread)

template <int ELEM>
__global__ __launch_bounds__(256, 2) void mx6_gemm_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                                                       const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws,
                                                       const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
                                                       int M, int N, int K, int tiles_n) {
  constexpr int FMT = ELEM == 3 ? 2 : 3;  // MFMA operand format: 2 = E2M3, 3 = E3M2
  constexpr int CPT = kChunks / 256;      // chunks per thread and operand
  __shared__ __attribute__((aligned(16))) uint8_t sa[kT * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t sw[kT * kPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves of 64 x 64 outputs
  // tile order as in the MX GEMM: each XCD takes a contiguous range of ids, and ids walk groups of 8
  // tile rows column by column, so that concurrent tiles share A and W rows in one L2
  const int tiles_m = (M + kT - 1) / kT;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  constexpr int GROUP = 8;
  const int group = (int)(id / (uint32_t)(GROUP * tiles_n));
  const int gsz = min(tiles_m - group * GROUP, GROUP);
  const int m0 = (group * GROUP + (int)(id % (uint32_t)gsz)) * kT;
  const int n0 = (int)((id % (uint32_t)(GROUP * tiles_n)) / (uint32_t)gsz) * kT;
  const int SK = K / 32;                  // blocks (and scale bytes) per row
  const size_t KB = (size_t)SK * 24;      // code bytes per row
  const int nstages = (SK + kStageBlocks - 1) / kStageBlocks;

  // scale of block b of a row; rows past M / N and blocks past K hold zero codes (any scale)
  auto scale = [&](const uint8_t* S, int grow, int rows, int b) {
    return (grow < rows && b < SK) ? (int)S[(size_t)grow * SK + b] : 127;
  };
  // stage s of an operand: rows x 96 bytes; chunk c = row c / 6, byte 16 (c % 6) of the row's
  // stage; blocks past K (the last stage of a K that is not a multiple of 128) load as zeros
  uint4 ra[CPT], rw[CPT];
  // scale bytes of the lane's rows for a stage: [tile][MFMA step], fetched a stage ahead with the codes
  int nsa[2][kStageBlocks / 2], nsw[2][kStageBlocks / 2];
  auto load = [&](int st) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u;
      const int row = c / 6, off = 16 * (c - 6 * (c / 6));
      const size_t kb = (size_t)st * kRowB + off;  // byte within the row
      ra[u] = uint4{0u, 0u, 0u, 0u};
      rw[u] = uint4{0u, 0u, 0u, 0u};
      if (kb < KB && m0 + row < M) ra[u] = *reinterpret_cast<const uint4*>(A + (size_t)(m0 + row) * KB + kb);
      if (kb < KB && n0 + row < N) rw[u] = *reinterpret_cast<const uint4*>(W + (size_t)(n0 + row) * KB + kb);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < kStageBlocks / 2; ++kk) {
        const int b = st * kStageBlocks + 2 * kk + q;
        nsa[t][kk] = scale(As, m0 + wm * 64 + 32 * t + r32, M, b);
        nsw[t][kk] = scale(Ws, n0 + wn * 64 + 32 * t + r32, N, b);
      }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u;
      const int row = c / 6, off = 16 * (c - 6 * (c / 6));
      uint2* da = reinterpret_cast<uint2*>(&sa[row * kPitch + off]);
      uint2* dw = reinterpret_cast<uint2*>(&sw[row * kPitch + off]);
      da[0] = make_uint2(ra[u].x, ra[u].y);
      da[1] = make_uint2(ra[u].z, ra[u].w);
      dw[0] = make_uint2(rw[u].x, rw[u].y);
      dw[1] = make_uint2(rw[u].z, rw[u].w);
    }
  };
  // lane (r, q) of an operand tile at MFMA step kk of the stage: block 2 kk + q, 24 bytes
  auto operand = [&](const uint8_t* s, int row, int kk) {
    const uint2* p = reinterpret_cast<const uint2*>(s + row * kPitch + 24 * (2 * kk + q));
    const uint2 x0 = p[0], x1 = p[1], x2 = p[2];
    return m6_v8i{(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y, (int)x2.x, (int)x2.y, 0, 0};
  };

  m6_v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = m6_v16f{};

  load(0);
  for (int st = 0; st < nstages; ++st) {
    __syncthreads();  // every wave is done reading the previous stage
    store();
    int csa[2][kStageBlocks / 2], csw[2][kStageBlocks / 2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < kStageBlocks / 2; ++kk) {
        csa[t][kk] = nsa[t][kk];
        csw[t][kk] = nsw[t][kk];
      }
    __syncthreads();
    if (st + 1 < nstages) load(st + 1);  // in flight while this stage computes
#pragma unroll
    for (int kk = 0; kk < kStageBlocks / 2; ++kk) {
      m6_v8i wop[2], aop[2];
      int wsc[2], asc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        aop[t] = operand(sa, wm * 64 + 32 * t + r32, kk);
        wop[t] = operand(sw, wn * 64 + 32 * t + r32, kk);
        asc[t] = csa[t][kk];
        wsc[t] = csw[t][kk];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[i], aop[j], acc[i][j], FMT, FMT, 0,
                                                                      wsc[i], 0, asc[j]);
      // one step's operands live at a time (keeps the kernel at two waves per SIMD)
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: lane (r32, q) of tile (i, j) holds output row m = m0 + wm 64 + 32 j + r32 and columns
  // n = n0 + wn 64 + 32 i + 8 g + 4 q + (0..3)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + 32 * j + r32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + 32 * i + 8 * g + 4 * q;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[u] = acc[i][j][4 * g + u];
          if (bias && n + u < N) v[u] += bf16_to_f32(bias[n + u]);
        }
        const m6_bf16x2 lo = __builtin_convertvector(m6_f32x2{v[0], v[1]}, m6_bf16x2);
        const m6_bf16x2 hi = __builtin_convertvector(m6_f32x2{v[2], v[3]}, m6_bf16x2);
        uint16_t* dst = out + (size_t)m * N + n;
        if ((N & 3) == 0 && n + 3 < N) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        } else {
          const uint32_t pl = __builtin_bit_cast(uint32_t, lo), ph = __builtin_bit_cast(uint32_t, hi);
          if (n < N) dst[0] = (uint16_t)pl;
          if (n + 1 < N) dst[1] = (uint16_t)(pl >> 16);
          if (n + 2 < N) dst[2] = (uint16_t)ph;
          if (n + 3 < N) dst[3] = (uint16_t)(ph >> 16);
        }
      }
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

hipError_t launch_mx6_gemm(int elem, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales, const uint16_t* bias, uint16_t* out,
                           hipStream_t stream) {
  const int64_t tiles_n = (N + kT - 1) / kT, tiles = ((M + kT - 1) / kT) * tiles_n;
  if (elem == 3)
    hipLaunchKernelGGL(mx6_gemm_kernel<3>, dim3((unsigned)tiles), dim3(256), 0, stream, a_codes, a_scales, w_codes,
                       w_scales, bias, out, (int)M, (int)N, (int)K, (int)tiles_n);
  else
    hipLaunchKernelGGL(mx6_gemm_kernel<4>, dim3((unsigned)tiles), dim3(256), 0, stream, a_codes, a_scales, w_codes,
                       w_scales, bias, out, (int)M, (int)N, (int)K, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace mxq
