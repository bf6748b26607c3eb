// Dynamic block-scaled quantizers for gfx950: MXFP8 / MXFP6 / MXFP4 (E8M0
// scale per 32 elements) and NVFP4-style (E4M3 scale per 16 elements + fp32
// tensor scale).  Method: aitrends.kr "Accelerating diffusion-model inference with
// MXFP8 and NVFP4 quantization on NVIDIA B200", Glossary ("Microscaling
// Formats", "MXFP8", "NVFP4") and "Section details" (dynamic activation
// quantization, dynamic per-tensor scale); encodings and the shared-exponent
// rule of the OCP Microscaling Formats v1.0 specification (which also defines
// the 6-bit E2M3 and E3M2 elements).
//
// Both quantizers are HBM-streaming kernels: every lane owns one 16-byte
// chunk (8 bf16) per iteration, loaded with one 128-bit load, so a wave reads
// 1 KiB of contiguous memory per instruction.  A 32-element MX block is four
// consecutive lanes (a DPP quad), a 16-element NVFP4 block two lanes; block
// maxima are exchanged with DPP quad permutes, no LDS.  The shared exponent
// comes from integer arithmetic on the bf16 bit patterns; MX element codes
// from the hardware bf16 -> FP8 / FP4 conversions, whose rounding was
// measured equal to the definition for every input (FP8 after a clamp, see
// below) and the bf16 -> FP6 conversions (measured exact, see
// mx_encode_fp6x8); NVFP4 codes, whose divisor is not a power of two, from
// exact comparisons against per-block thresholds.
#include "mx_encode.h"
#include "mxq_internal.h"

namespace mxq {
namespace {

__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {  // lanes 0<->1, 2<->3 of each quad
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {  // lanes 0<->2, 1<->3 of each quad
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_next(uint32_t v) {  // lane t of each quad gets lane min(t + 1, 3)
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xF9, 0xF, 0xF, false);
}

// Largest |x| (as bf16 magnitude bits) of the 8 elements in a 16-byte chunk.
__device__ __forceinline__ uint32_t chunk_absmax_bits(const uint4& v) {
  return max(mx_absmax_bits4(v.x, v.y), mx_absmax_bits4(v.z, v.w));
}

// Loads in flight per lane: each lane issues kBatch independent 16-byte loads
// (grid-stride apart) before processing them, so that a CU keeps enough bytes
// in flight to cover HBM latency; the stride is a multiple of 256 chunks, so
// block-aligned lane groups stay aligned.
constexpr int kBatch = 4;

// Calls f(v, i) for every chunk i < nchunks of this lane, kBatch loads at a
// time.  `i < nchunks` is uniform over any lane group whose chunks share a
// block, because nchunks is a multiple of the group size.
template <typename F>
__device__ __forceinline__ void for_chunks(const uint4* __restrict__ x, int64_t nchunks, F&& f) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < nchunks; i0 += stride * kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = i < nchunks ? x[i] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < nchunks) f(v[u], i);
    }
  }
}

// Byte offset of the scale of block b (row-major block index, srow blocks per
// row).  PKS == 0: b itself.  PKS == 1: the packed layout the MX GEMM stages
// from: rows in groups of 32, each group's scales stage-major with P blocks
// per row and stage (P = 4: 128 elements of FP8 / FP6; P = 8: 256 elements of
// FP4), so that one stage's scales of 32 rows are 32 P contiguous bytes.  The
// host keeps the block count below 2^32 for PKS == 1 and passes the row
// division as a multiply: row = (t + ((b - t) >> 1)) >> dsh with
// t = umulhi(b, dmul), exact for every 32-bit b (the round-up method for
// unsigned division by an invariant integer, Granlund and Montgomery).
struct RowDiv {
  uint32_t srow, dmul, dsh;
};
template <int P, int PKS>
__device__ __forceinline__ size_t scale_offset(int64_t b, const RowDiv& rd) {
  if constexpr (PKS == 0) {
    return (size_t)b;
  } else {
    const uint32_t b32 = (uint32_t)b;
    const uint32_t t = __umulhi(b32, rd.dmul);
    const uint32_t row = (t + ((b32 - t) >> 1)) >> rd.dsh, kb = b32 - row * rd.srow;
    return (size_t)(row / 32u) * 32u * rd.srow + (kb / P) * (32u * P) + (row % 32u) * P + kb % P;
  }
}

// Multiplier and shift of the row division for srow >= 2 blocks per row:
// l = ceil(log2 srow), dmul = floor(2^32 (2^l - srow) / srow) + 1, dsh = l - 1.
inline RowDiv row_div(uint32_t srow) {
  uint32_t l = 0;
  while ((1ull << l) < srow) ++l;
  const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - srow)) / srow + 1;
  return RowDiv{srow, (uint32_t)m, l - 1};
}

// One lane = one 16-byte chunk (8 consecutive bf16); four lanes = one
// 32-element block.  nchunks is a multiple of 4 and every quad of lanes
// starts on a block boundary, so the whole quad is active together.
template <int ELEM, int PKS>
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint4* __restrict__ x, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t nchunks,
                                                       int rceil, RowDiv rd) {
  for_chunks(x, nchunks, [&](const uint4& v, int64_t i) {
    uint32_t m = chunk_absmax_bits(v);
    m = max(m, quad_swap1(m));
    m = max(m, quad_swap2(m));

    uint32_t scale_byte;
    uint32_t lo = 0, hi = 0;  // FP8: codes 0-3, 4-7; FP4: lo = codes 0-7
    if (m >= 0x7F80u) {  // NaN or Inf in the block: NaN scale, zero codes
      scale_byte = 0xFFu;
    } else {
      const int e = mx_shared_exponent<ELEM>(m, rceil);
      scale_byte = (uint32_t)(e + 127);
      if constexpr (ELEM == 1) {
        lo = mx_encode_fp8x4(v.x, v.y, e);
        hi = mx_encode_fp8x4(v.z, v.w, e);
      } else {
        lo = mx_encode_fp4x4<0>(0u, v.x, v.y, e);
        lo = mx_encode_fp4x4<2>(lo, v.z, v.w, e);
      }
    }
    if (ELEM == 1) reinterpret_cast<uint2*>(codes)[i] = make_uint2(lo, hi);
    else reinterpret_cast<uint32_t*>(codes)[i] = lo;
    if ((i & 3) == 0) scales[scale_offset<ELEM == 1 ? 4 : 8, PKS>(i >> 2, rd)] = (uint8_t)scale_byte;
  });
}


// ----------------------------------------------------------------- MXFP6
// MXFP6 codes: each 32-element block is a 32-byte slot holding its 192-bit
// code integer (element j at bits 6j, little-endian) and 8 zero bytes.  Lane
// t of a quad encodes elements 8t .. 8t+7, i.e. bits 48t .. 48t+47 of the
// integer (p_t); the slot's 8-byte word t is bits 64t .. 64t+63, which is
// (p_t >> 16t) | (p_{t+1} << (48 - 16t)) for t < 3 and zero for t = 3, so
// one quad shift hands each lane its neighbour's bits and every lane stores
// one word (a wave writes 512 contiguous bytes).
template <int ELEM, int PKS>
__global__ __launch_bounds__(256) void mx6_quant_kernel(const uint4* __restrict__ x, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, int64_t nchunks, int rceil,
                                                        RowDiv rd) {
  for_chunks(x, nchunks, [&](const uint4& v, int64_t i) {
    uint32_t m = chunk_absmax_bits(v);
    m = max(m, quad_swap1(m));
    m = max(m, quad_swap2(m));
    uint32_t lo = 0, hi = 0;
    uint32_t scale_byte = 0xFFu;  // NaN or Inf in the block: NaN scale, zero codes
    if (m < 0x7F80u) {
      const int e = mx_shared_exponent<ELEM>(m, rceil);
      scale_byte = (uint32_t)(e + 127);
      mx_encode_fp6x8<ELEM>(v.x, v.y, v.z, v.w, e, lo, hi);
    }
    const uint64_t p = ((uint64_t)hi << 32) | lo;
    const uint32_t t = (uint32_t)i & 3u;
    const uint64_t pn = ((uint64_t)quad_next(hi) << 32) | quad_next(lo);
    const uint64_t word = t == 3u ? 0ull : (p >> (16 * t)) | (pn << (48 - 16 * t));
    reinterpret_cast<uint64_t*>(codes)[i] = word;
    if (t == 0u) scales[scale_offset<4, PKS>(i >> 2, rd)] = (uint8_t)scale_byte;
  });
}

// ----------------------------------------------------------------- NVFP4

constexpr int kNvPartialsMax = 1024;

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Phase 1: per-workgroup maxima of the bf16 magnitude bits.
__global__ __launch_bounds__(256) void absmax_partials_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                              uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  for_chunks(x, nchunks, [&](const uint4& v, int64_t) { m = max(m, chunk_absmax_bits(v)); });
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// E4M3 code of a positive, finite double q (nearest even, saturating at 448).
__device__ __forceinline__ uint32_t e4m3_encode_pos(double q) {
  if (q >= 448.0) return 0x7Eu;
  const uint64_t u = (uint64_t)__double_as_longlong(q);
  const int E = (int)((u >> 52) & 0x7FF) - 1023;
  if (E >= -6) {
    const uint64_t mant = u & 0xFFFFFFFFFFFFFull;
    uint32_t c = ((uint32_t)(E + 7) << 3) | (uint32_t)(mant >> 49);
    const uint64_t rem = mant & ((1ull << 49) - 1);
    const uint64_t half = 1ull << 48;
    c += (rem > half || (rem == half && (c & 1u))) ? 1u : 0u;
    return c;
  }
  return (uint32_t)rint(q * 512.0);  // subnormal grid step 2^-9; rint rounds half to even
}

__device__ __forceinline__ double e4m3_decode_pos(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xF, m = c & 7;
  if (e == 0) return (double)m * 0x1p-9;
  return (double)__uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Smallest float32 bit pattern V such that, for a non-negative float32 |x|,
// |x| >= V holds exactly when |x| is above the midpoint T, or equal to it and
// the tie goes up (tie_up).  U = T rounded up to float32; if T is a float32,
// a tie that goes down needs |x| > T, i.e. |x| >= next float after T.
__device__ __forceinline__ uint32_t midpoint_threshold(double T, bool tie_up) {
  const float f = (float)T;
  uint32_t ub = __float_as_uint(f);
  if ((double)f < T) ub += 1u;
  const bool exact = (double)__uint_as_float(ub) == T;
  return (exact && !tie_up) ? ub + 1u : ub;
}

// Threshold from exact fp32 arithmetic: T = a * ts with a = t * dec(sc) exact
// in fp32 (at most 7 significant bits).  p = RN(T) and the FMA residual
// e = T - p (exact while T's lowest bit stays a normal fp32, which holds for
// ts >= 2^-60) decide the smallest float >= T: p when T < p, the next float
// when T > p, and when T = p either p (tie goes up) or the next float.
__device__ __forceinline__ uint32_t midpoint_threshold_f32(float a, float ts, bool tie_up) {
  const float p = a * ts;
  const float e = __builtin_fmaf(a, ts, -p);
  const uint32_t pb = __float_as_uint(p);
  return (e > 0.0f || (e == 0.0f && !tie_up)) ? pb + 1u : pb;
}

// E2M1 code magnitudes (0..7) of 8 bf16 values against the 7 thresholds,
// with the sign bit of each input kept, packed 4 bits per element (element j
// in bits 4j .. 4j + 3).
__device__ __forceinline__ uint32_t e2m1_codes8(const uint4& v, const uint32_t (&V)[7], bool keep_sign) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
    const uint32_t a = (h & 0x7FFFu) << 16;  // |x| as float32 bits
    uint32_t k = 0;
#pragma unroll
    for (int t = 0; t < 7; ++t) k += (a >= V[t]) ? 1u : 0u;
    if (keep_sign) k |= (h >> 12) & 8u;
    o |= k << (4 * j);
  }
  return o;
}

// Phase 2: one lane per 16-element block (two 16-byte chunks): block scale,
// thresholds, element codes.
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                          float* __restrict__ ts_out,
                                                          const uint32_t* __restrict__ partials, int npartials) {
  __shared__ uint32_t red[4];
  uint32_t g = 0;
  for (int j = threadIdx.x; j < npartials; j += 256) g = max(g, partials[j]);
  g = wave_max(g);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = g;
  __syncthreads();
  g = max(max(red[0], red[1]), max(red[2], red[3]));

  const bool nonfinite = g >= 0x7F80u;
  float ts;
  if (nonfinite) {
    ts = __uint_as_float(0x7FC00000u);
  } else if (g == 0) {
    ts = 1.0f;
  } else {
    // G / 2688 in double is correctly rounded; its float32 rounding is then the
    // correctly rounded quotient: G has 8 significant bits and 2688 = 2^7 * 21,
    // so the exact quotient is either short or has a binary expansion of
    // period <= 6, never within 2^-53 of a float32 rounding midpoint.
    ts = (float)((double)bf16_to_f32(g) / 2688.0);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = ts;
  const double ts64 = (double)ts;
  const bool fast = !nonfinite && ts >= 0x1p-60f;  // uniform

  const int64_t nblocks = nchunks / 2;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b0 = (int64_t)blockIdx.x * 256 + threadIdx.x; b0 < nblocks; b0 += stride * kBatch) {
    uint4 v[kBatch][2];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t b = b0 + u * stride;
      if (b < nblocks) {
        v[u][0] = x[2 * b];
        v[u][1] = x[2 * b + 1];
      } else {
        v[u][0] = v[u][1] = uint4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t b = b0 + u * stride;
      if (b >= nblocks) continue;
      const uint32_t bm = max(chunk_absmax_bits(v[u][0]), chunk_absmax_bits(v[u][1]));
      uint32_t sc;
      uint32_t V[7];
      if (nonfinite || bm == 0) {
        sc = nonfinite ? 0x7Fu : 0u;
#pragma unroll
        for (int j = 0; j < 7; ++j) V[j] = 0xFFFFFFFFu;
      } else {
        // block scale: one rounding of B / (6 ts); operands exact in double and
        // the division correctly rounded, so the E4M3 rounding sees the exact
        // quotient's decisions (a non-tie quotient is >= ~2^-32 relative away
        // from any E4M3 midpoint).
        const double q = (double)bf16_to_f32(bm) / (6.0 * ts64);
        sc = e4m3_encode_pos(q);
        if (sc == 0) sc = 1;
        // E2M1 midpoints between codes j and j+1 (0.25 .. 5 times the scale);
        // ties go to the even code, i.e. up after odd codes.
        if (fast) {
          const float d = (float)e4m3_decode_pos(sc);  // exact
          V[0] = midpoint_threshold_f32(0.25f * d, ts, false);
          V[1] = midpoint_threshold_f32(0.75f * d, ts, true);
          V[2] = midpoint_threshold_f32(1.25f * d, ts, false);
          V[3] = midpoint_threshold_f32(1.75f * d, ts, true);
          V[4] = midpoint_threshold_f32(2.5f * d, ts, false);
          V[5] = midpoint_threshold_f32(3.5f * d, ts, true);
          V[6] = midpoint_threshold_f32(5.0f * d, ts, false);
        } else {
          const double s = e4m3_decode_pos(sc) * ts64;  // <= 28 significant bits: exact
          // t * s has <= 31 significant bits: exact in double
          V[0] = midpoint_threshold(0.25 * s, false);
          V[1] = midpoint_threshold(0.75 * s, true);
          V[2] = midpoint_threshold(1.25 * s, false);
          V[3] = midpoint_threshold(1.75 * s, true);
          V[4] = midpoint_threshold(2.5 * s, false);
          V[5] = midpoint_threshold(3.5 * s, true);
          V[6] = midpoint_threshold(5.0 * s, false);
        }
      }
      const uint32_t lo = e2m1_codes8(v[u][0], V, !nonfinite);
      const uint32_t hi = e2m1_codes8(v[u][1], V, !nonfinite);
      reinterpret_cast<uint2*>(codes)[b] = make_uint2(lo, hi);
      scales[b] = (uint8_t)sc;
    }
  }
}

int grid_for(int64_t nchunks, int64_t cap) {
  int64_t g = (nchunks + 255) / 256;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

template <int PKS>
void launch_mx_quant_pks(int elem, int grid, hipStream_t stream, const uint4* xv, uint8_t* codes, uint8_t* scales,
                         int64_t nchunks, int rceil, RowDiv rd) {
  if (elem == 1)
    hipLaunchKernelGGL((mx_quant_kernel<1, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nchunks, rceil,
                       rd);
  else if (elem == 2)
    hipLaunchKernelGGL((mx_quant_kernel<2, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nchunks, rceil,
                       rd);
  else if (elem == 3)
    hipLaunchKernelGGL((mx6_quant_kernel<3, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nchunks,
                       rceil, rd);
  else
    hipLaunchKernelGGL((mx6_quant_kernel<4, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nchunks,
                       rceil, rd);
}

hipError_t launch_mx_quant(int elem, int rceil, int packed, const uint16_t* x, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) return hipSuccess;
  const int grid = grid_for((nchunks + kBatch - 1) / kBatch, 8192);
  const uint4* xv = (const uint4*)x;
  // packed scales need whole 128- or 256-element stages per row, so srow >= 4
  const RowDiv rd = packed ? row_div((uint32_t)(cols / 32)) : RowDiv{(uint32_t)(cols / 32), 0u, 0u};
  if (packed) launch_mx_quant_pks<1>(elem, grid, stream, xv, codes, scales, nchunks, rceil, rd);
  else launch_mx_quant_pks<0>(elem, grid, stream, xv, codes, scales, nchunks, rceil, rd);
  return hipGetLastError();
}

int64_t nvfp4_partials_count(int64_t n_elems) {
  const int64_t nchunks = n_elems / 8;
  int64_t p = (nchunks + 2047) / 2048;  // >= 8 chunks per lane before capping
  if (p > kNvPartialsMax) p = kNvPartialsMax;
  if (p < 1) p = 1;
  return p;
}

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              float* tensor_scale, uint32_t* partials, hipStream_t stream) {
  const int64_t nchunks = rows * cols / 8;
  const int P = (int)nvfp4_partials_count(rows * cols);
  hipLaunchKernelGGL(absmax_partials_kernel, dim3(P), dim3(256), 0, stream, (const uint4*)x, nchunks, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = grid_for((nchunks / 2 + kBatch - 1) / kBatch, 4096);
  hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(grid), dim3(256), 0, stream, (const uint4*)x, nchunks, codes, scales,
                     tensor_scale, (const uint32_t*)partials, P);
  return hipGetLastError();
}

}  // namespace mxq
