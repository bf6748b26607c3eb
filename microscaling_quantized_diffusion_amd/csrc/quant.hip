// Dynamic block-scaled quantizers for gfx950: MXFP8 / MXFP6 / MXFP4 (E8M0
// scale per 32 elements) and NVFP4-style (E4M3 scale per 16 elements + fp32
// tensor scale).  Method: aitrends.kr "Accelerating diffusion-model inference with
// MXFP8 and NVFP4 quantization on NVIDIA B200", Glossary ("Microscaling
// Formats", "MXFP8", "NVFP4") and "Section details" (dynamic activation
// quantization, dynamic per-tensor scale); encodings and the shared-exponent
// rule of the OCP Microscaling Formats v1.0 specification (which also defines
// the 6-bit E2M3 and E3M2 elements).
//
// Both quantizers are HBM-streaming kernels in which one lane owns one block
// (MX: 32 elements, four 16-byte chunks, 64 contiguous bytes; NVFP4: 16
// elements, two chunks); the longer NVFP4 encoder loads the next block of the
// lane's grid-stride sequence before it encodes the current one.  The shared exponent comes from integer arithmetic on the bf16
// bit patterns; MX element codes from the hardware bf16 -> FP8 / FP4 / FP6
// conversions, whose rounding was measured equal to the definition for
// every input (FP8 after a clamp, see mx_encode.h).  NVFP4 codes, whose
// divisor is not a power of two, are the number of the block's seven E2M1
// midpoint thresholds at or below |x|: one read of a per-workgroup byte table
// of the scale code's significand class (or, for tiny tensor scales, a
// search over the thresholds themselves).
#include "mx_encode.h"
#include "mxq_internal.h"

namespace mxq {
namespace {

// Largest |x| (as bf16 magnitude bits) of the 8 elements in a 16-byte chunk.
__device__ __forceinline__ uint32_t chunk_absmax_bits(const uint4& v) {
  return max(mx_absmax_bits4(v.x, v.y), mx_absmax_bits4(v.z, v.w));
}

// Loads in flight per lane in the global-maximum pass: each lane issues
// kBatch independent 16-byte loads (grid-stride apart) before taking their
// maxima, so that a CU keeps enough bytes in flight to cover HBM latency.
constexpr int kBatch = 4;

// Calls f(v, i) for every chunk i < nchunks of this lane, kBatch loads at a
// time.
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

// Calls encode(b, v) for every block b < nblocks of this lane's grid-stride
// sequence, v holding the block's CH 16-byte chunks.
template <int CH, typename F>
__device__ __forceinline__ void for_blocks(const uint4* __restrict__ x, int64_t nblocks, F&& encode) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += stride) {
    uint4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = x[CH * b + c];
    encode(b, v);
  }
}

// The same, with the next block's loads issued before the current block is
// encoded (for encoders long enough to hide them behind).
template <int CH, typename F>
__device__ __forceinline__ void for_blocks_prefetched(const uint4* __restrict__ x, int64_t nblocks, F&& encode) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  auto load = [&](int64_t b, uint4 (&v)[CH]) {
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = b < nblocks ? x[CH * b + c] : uint4{0u, 0u, 0u, 0u};
  };
  int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 va[CH], vb[CH];
  load(b, va);
  while (b < nblocks) {
    load(b + stride, vb);
    encode(b, va);
    b += stride;
    if (b >= nblocks) break;
    load(b + stride, va);
    encode(b, vb);
    b += stride;
  }
}

// One lane = one 32-element block (four chunks, 64 contiguous bytes): its
// largest magnitude, shared exponent, element codes and scale byte.  Codes:
// FP8 32 bytes, FP4 16 bytes, FP6 a 32-byte slot holding the block's 192-bit
// code integer (element j at bits 6 j, little-endian) and 8 zero bytes.
template <int ELEM, int PKS>
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint4* __restrict__ x, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t nblocks, int rceil,
                                                       RowDiv rd) {
  for_blocks<4>(x, nblocks, [&](int64_t b, const uint4 (&v)[4]) {
    const uint32_t m = max(max(chunk_absmax_bits(v[0]), chunk_absmax_bits(v[1])),
                           max(chunk_absmax_bits(v[2]), chunk_absmax_bits(v[3])));
    const bool nonfinite = m >= 0x7F80u;  // NaN or Inf in the block: NaN scale, zero codes
    const int e = nonfinite ? 0 : mx_shared_exponent<ELEM>(m, rceil);
    const uint32_t keep = nonfinite ? 0u : 0xFFFFFFFFu;
    if constexpr (ELEM == 1) {
      uint32_t c[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[2 * k] = mx_encode_fp8x4(v[k].x, v[k].y, e) & keep;
        c[2 * k + 1] = mx_encode_fp8x4(v[k].z, v[k].w, e) & keep;
      }
      uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    } else if constexpr (ELEM == 2) {
      uint32_t c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        c[k] = mx_encode_fp4x4<2>(mx_encode_fp4x4<0>(0u, v[k].x, v[k].y, e), v[k].z, v[k].w, e) & keep;
      *reinterpret_cast<uint4*>(codes + 16 * b) = make_uint4(c[0], c[1], c[2], c[3]);
    } else {
      uint32_t r[6];
      mx_encode_fp6x32<ELEM>(v, e, r);
      uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
      dst[0] = make_uint4(r[0] & keep, r[1] & keep, r[2] & keep, r[3] & keep);
      dst[1] = make_uint4(r[4] & keep, r[5] & keep, 0u, 0u);
    }
    scales[scale_offset<ELEM == 2 ? 8 : 4, PKS>(b, rd)] = nonfinite ? 0xFFu : (uint8_t)(e + 127);
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

// The seven E2M1 midpoint thresholds (0.25 .. 5 times the block scale
// dec(sc) * ts) as float32 bit patterns V: |x| rounds above midpoint t
// exactly when |x| >= V[t].  Ties go to the even code, i.e. up after odd
// codes.
__device__ __forceinline__ void nv_thresholds(uint32_t sc, float ts, double ts64, bool fast, uint32_t (&V)[7]) {
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

// A float32 threshold V as the smallest bf16 magnitude pattern h with
// (h << 16) >= V, which decides every bf16 |x| the same way, capped at 0x8000
// (above every magnitude pattern), in both 16-bit halves.
__device__ __forceinline__ uint32_t thr16x2(uint32_t V) {
  uint32_t c = (V >> 16) + ((V & 0xFFFFu) != 0u ? 1u : 0u);
  c = min(c, 0x8000u);
  return c | (c << 16);
}

typedef unsigned short nv_u16x2 __attribute__((ext_vector_type(2)));
typedef short nv_s16x2 __attribute__((ext_vector_type(2)));
// 0xFFFF in each 16-bit half where a < t, else 0 (a, t <= 0x8000 in each
// half, so the sign of the 16-bit difference decides): one packed subtract
// and one packed arithmetic shift, the shift count in a register for both
// halves.
__device__ __forceinline__ uint32_t lt_mask16x2(uint32_t a, uint32_t t) {
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_bit_cast(nv_u16x2, a) - __builtin_bit_cast(nv_u16x2, t));
  uint32_t m;
  asm("v_pk_ashrrev_i16 %0, %1, %2" : "=v"(m) : "v"(0x000F000Fu), "v"(d));
  return m;
}
__device__ __forceinline__ uint32_t sel_mask(uint32_t m, uint32_t x, uint32_t y) { return (m & x) | (~m & y); }

// Two bf16 (one dword) -> their E2M1 codes in bits 0..3 and 16..19: the
// magnitude is the number of thresholds T[0..6] (packed, sorted) at or below
// |x|, found by a three-level search; signmask keeps the sign bits.
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t w, const uint32_t (&T)[7], uint32_t signmask) {
  const uint32_t a = w & 0x7FFF7FFFu;
  const uint32_t m1 = lt_mask16x2(a, T[3]);
  const uint32_t m2 = lt_mask16x2(a, sel_mask(m1, T[1], T[5]));
  const uint32_t m3 = lt_mask16x2(a, sel_mask(m1, sel_mask(m2, T[0], T[2]), sel_mask(m2, T[4], T[6])));
  const uint32_t k = ((m1 & 0x00040004u) | (m2 & 0x00020002u) | (m3 & 0x00010001u)) ^ 0x00070007u;
  return k | ((w >> 12) & signmask);
}
// Eight bf16 (one chunk) -> eight E2M1 codes, element j in bits 4 j .. 4 j + 3.
__device__ __forceinline__ uint32_t e2m1_codes8(const uint4& v, const uint32_t (&T)[7], uint32_t signmask) {
  uint32_t u0 = e2m1_pair(v.x, T, signmask), u1 = e2m1_pair(v.y, T, signmask);
  uint32_t u2 = e2m1_pair(v.z, T, signmask), u3 = e2m1_pair(v.w, T, signmask);
  u0 |= u0 >> 12;  // byte 0: the pair's two codes
  u1 |= u1 >> 12;
  u2 |= u2 >> 12;
  u3 |= u3 >> 12;
  return (u0 & 0xFFu) | ((u1 & 0xFFu) << 8) | ((u2 & 0xFFu) << 16) | (u3 << 24);
}

// Class tables.  dec(c) = 2^E d with d in [1, 2) one of eight significands
// (1 + k / 8), so for ts >= 2^-60 (every threshold a normal float32 and bf16)
// the seven thresholds of code c are those of the representative code
// 0x38 | k (dec = d) shifted by E in the bf16 exponent field: T_j(c) =
// T_j(0x38 | k) + 128 E, since rounding, the FMA residual and the round-up to
// bf16 all commute with scaling by 2^E there.  So the E2M1 magnitude of a bf16
// |x| under code c is tab_k[min(sat(|x| - (T_0(c) - 1)), kNvTab - 1)] with
// tab_k[i] = #{j : T_j(0x38 | k) - T_0(0x38 | k) < i}: one byte-table read per
// element in place of the threshold search.
constexpr int kNvTab = 640;  // bytes per class table (T_6 - T_0 <= 4.33 binades = 555 bf16 steps)

typedef unsigned short nv_us2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(nv_us2, a), __builtin_bit_cast(nv_us2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_min(__builtin_bit_cast(nv_us2, a), __builtin_bit_cast(nv_us2, b)));
}
// max(a - b, 0) in each 16-bit half
__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(nv_us2, a),
                                                                    __builtin_bit_cast(nv_us2, b)));
}

// Phase 2: one lane per 16-element block (two chunks).  Every workgroup first
// takes the global maximum from the partials and builds its tables in LDS
// from the tensor scale ts:
//   up[c]   the smallest bf16 magnitude pattern B whose block scale B / (6 ts)
//           rounds (nearest even E4M3, saturating at 448) to a code above c;
//   for ts >= 2^-60: the eight class tables, and per code c the offset
//           T_0(c) - 1 and its class;
//   otherwise (and should a class-table check fail): thr[c], the seven
//           packed element thresholds of code c (c = 0 and 0x7F: above every
//           magnitude), searched per element.
// A block's scale code is then the hardware E4M3 rounding of the float32
// estimate bm * fl(1 / (6 ts)), whose relative error (a few units of 2^-24)
// moves it by at most one code, corrected exactly against up[c0 - 1] and
// up[c0]; below ts = 2^-60 the estimate is not used and a binary search over
// up[] finds the code.  A nonzero block's code is at least 1.
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint4* __restrict__ x, int64_t nchunks,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                          float* __restrict__ ts_out,
                                                          const uint32_t* __restrict__ partials, int npartials) {
  __shared__ uint32_t red[4];
  __shared__ uint4 thr[128][2];
  __shared__ uint16_t up[128];
  __shared__ uint32_t fix[128];    // up[c - 1] (0 for c = 0) | up[c] << 16
  __shared__ uint32_t cinfo[128];  // T_0(c) - 1 | class table offset << 16
  __shared__ uint16_t rep[8][8];   // T_0 .. T_6 of the representative codes 0x38 | k
  __shared__ __attribute__((aligned(16))) uint8_t ctab[8 * kNvTab];
  __shared__ uint32_t tab_bad;
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
  const int t = threadIdx.x;

  if (t < 128) {
    uint32_t u = 0x8000u;
    if (t < 0x7E && !nonfinite) {
      // midpoint of codes t and t + 1 (<= 5 significant bits) times 6 ts: exact in double
      const double mid = 0.5 * (e4m3_decode_pos((uint32_t)t) + e4m3_decode_pos((uint32_t)t + 1u));
      const uint32_t V = midpoint_threshold(mid * 6.0 * ts64, ((t + 1) & 1) == 0);
      u = thr16x2(V) & 0xFFFFu;
    }
    up[t] = (uint16_t)u;
  }
  if (t == 0) tab_bad = fast ? 0u : 1u;
  if (fast && t < 8) {
    uint32_t V[7];
    nv_thresholds(0x38u | (uint32_t)t, ts, ts64, true, V);
#pragma unroll
    for (int j = 0; j < 7; ++j) rep[t][j] = (uint16_t)(thr16x2(V[j]) & 0xFFFFu);
  }
  __syncthreads();
  if (t < 128) fix[t] = (t ? (uint32_t)up[t - 1] : 0u) | ((uint32_t)up[t] << 16);
  if (fast) {
    if (t < 128) {
      uint32_t ci = 0x7FFFu;  // codes 0 and 0x7F: every magnitude maps to entry 0, code 0
      if (t != 0 && t != 0x7F) {
        const float d = (float)e4m3_decode_pos((uint32_t)t);  // exact
        const uint32_t k = (__float_as_uint(d) >> 20) & 7u;
        const uint32_t t0 = thr16x2(midpoint_threshold_f32(0.25f * d, ts, false)) & 0xFFFFu;
        const uint32_t t6 = thr16x2(midpoint_threshold_f32(5.0f * d, ts, false)) & 0xFFFFu;
        if (t6 - t0 != (uint32_t)rep[k][6] - (uint32_t)rep[k][0]) tab_bad = 1u;
        ci = (t0 - 1u) | ((k * (uint32_t)kNvTab) << 16);
      }
      cinfo[t] = ci;
    }
    if (t < 8) {
      // at most one step in any 20 consecutive entries, and the last entry is 7
#pragma unroll
      for (int j = 0; j < 6; ++j)
        if ((int)rep[t][j + 1] - (int)rep[t][j] < kNvTab / 32 + 1) tab_bad = 1u;
      if ((int)rep[t][6] - (int)rep[t][0] > kNvTab - 2) tab_bad = 1u;
    }
    // thread t fills entries s .. s + 19 of class k's table
    const int k = t >> 5, s = (t & 31) * (kNvTab / 32);
    const int r0 = rep[k][0];
    uint32_t v0 = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) v0 += ((int)rep[k][j] - r0 < s) ? 1u : 0u;
    const int nxt = v0 < 7 ? (int)rep[k][v0] - r0 + 1 : (1 << 20);  // first entry above the next threshold
    uint32_t* dst = reinterpret_cast<uint32_t*>(ctab + k * kNvTab + s);
#pragma unroll
    for (int dd = 0; dd < kNvTab / 128; ++dd) {
      const int q = nxt - (s + 4 * dd);
      const uint32_t step = q <= 0 ? 0x01010101u : q >= 4 ? 0u : (0x01010101u << (8 * q));
      dst[dd] = v0 * 0x01010101u + step;
    }
  }
  __syncthreads();
  const bool table = __builtin_amdgcn_readfirstlane(tab_bad) == 0u;  // uniform: implies fast

  const float inv6ts = 1.0f / (6.0f * ts);
  // the block's scale code from its largest magnitude bm (fast: estimate and
  // exact correction; otherwise the binary search over up[])
  auto scale_code = [&](uint32_t bm) {
    uint32_t c = 0;
    if (nonfinite) {
      c = 0x7Fu;
    } else if (bm != 0) {
      if (fast) {
        const float qf = fminf(bf16_to_f32(bm) * inv6ts, 448.0f);
        const uint32_t c0 =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(nv_s16x2{0, 0}, qf, qf, 1.0f, false)) &
            0x7Fu;
        const uint32_t f = fix[c0];
        c = c0 + (bm >= (f >> 16) ? 1u : 0u) - (bm < (f & 0xFFFFu) ? 1u : 0u);
      } else {
#pragma unroll
        for (uint32_t step = 64; step >= 1; step >>= 1)
          if (c + step <= 0x7Eu && bm >= up[c + step - 1]) c += step;
      }
      c = max(c, 1u);
    }
    return c;
  };

  if (table) {
    constexpr uint32_t kCap2 = (uint32_t)(kNvTab - 1) * 0x10001u;
    for_blocks_prefetched<2>(x, nchunks / 2, [&](int64_t b, const uint4 (&v)[2]) {
      const uint32_t w[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
      uint32_t a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = w[i] & 0x7FFF7FFFu;
      const uint32_t m = pk_max_u16(pk_max_u16(pk_max_u16(a[0], a[1]), pk_max_u16(a[2], a[3])),
                                    pk_max_u16(pk_max_u16(a[4], a[5]), pk_max_u16(a[6], a[7])));
      const uint32_t c = scale_code(max(m & 0xFFFFu, m >> 16));
      const uint32_t ci = cinfo[c];
      const uint32_t base2 = (ci & 0xFFFFu) * 0x10001u;
      const uint8_t* tb = ctab + (ci >> 16);
      uint32_t out[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t u[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t d = pk_min_u16(pk_sub_sat_u16(a[4 * h + p], base2), kCap2);
          // codes in bits 0..3 and 16..19 with their signs, then byte 0 holds both
          uint32_t e = (uint32_t)tb[d & 0xFFFFu] | ((uint32_t)tb[d >> 16] << 16) | ((w[4 * h + p] >> 12) & 0x00080008u);
          u[p] = e | (e >> 12);
        }
        out[h] = (u[0] & 0xFFu) | ((u[1] & 0xFFu) << 8) | ((u[2] & 0xFFu) << 16) | (u[3] << 24);
      }
      reinterpret_cast<uint2*>(codes)[b] = make_uint2(out[0], out[1]);
      scales[b] = (uint8_t)c;
    });
    return;
  }

  {
    const int c = t >> 1;  // thread pair 2c, 2c + 1 fills thr[c]
    uint32_t V[7];
    if (c == 0 || c == 0x7F || nonfinite) {
#pragma unroll
      for (int j = 0; j < 7; ++j) V[j] = 0xFFFFFFFFu;
    } else {
      nv_thresholds((uint32_t)c, ts, ts64, fast, V);
    }
    if ((t & 1) == 0) thr[c][0] = make_uint4(thr16x2(V[0]), thr16x2(V[1]), thr16x2(V[2]), thr16x2(V[3]));
    else thr[c][1] = make_uint4(thr16x2(V[4]), thr16x2(V[5]), thr16x2(V[6]), 0x80008000u);
  }
  __syncthreads();

  const uint32_t signmask = nonfinite ? 0u : 0x00080008u;
  for_blocks_prefetched<2>(x, nchunks / 2, [&](int64_t b, const uint4 (&v)[2]) {
    const uint32_t c = scale_code(max(chunk_absmax_bits(v[0]), chunk_absmax_bits(v[1])));
    const uint4 T0 = thr[c][0], T1 = thr[c][1];
    const uint32_t T[7] = {T0.x, T0.y, T0.z, T0.w, T1.x, T1.y, T1.z};
    reinterpret_cast<uint2*>(codes)[b] = make_uint2(e2m1_codes8(v[0], T, signmask), e2m1_codes8(v[1], T, signmask));
    scales[b] = (uint8_t)c;
  });
}

int grid_for(int64_t nlanes, int64_t cap) {
  int64_t g = (nlanes + 255) / 256;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

template <int PKS>
void launch_mx_quant_pks(int elem, int grid, hipStream_t stream, const uint4* xv, uint8_t* codes, uint8_t* scales,
                         int64_t nblocks, int rceil, RowDiv rd) {
  if (elem == 1)
    hipLaunchKernelGGL((mx_quant_kernel<1, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nblocks, rceil,
                       rd);
  else if (elem == 2)
    hipLaunchKernelGGL((mx_quant_kernel<2, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nblocks, rceil,
                       rd);
  else if (elem == 3)
    hipLaunchKernelGGL((mx_quant_kernel<3, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nblocks, rceil,
                       rd);
  else
    hipLaunchKernelGGL((mx_quant_kernel<4, PKS>), dim3(grid), dim3(256), 0, stream, xv, codes, scales, nblocks, rceil,
                       rd);
}

// Workgroups per launch: one block per lane up to the cap, beyond it a
// grid-stride sequence of blocks per lane (measured on the FLUX activations:
// 1024 workgroups for the 32-element MX blocks, 2048 for the NVFP4 pass).
constexpr int64_t kMxGridCap = 1024;
constexpr int64_t kNvGridCap = 2048;

hipError_t launch_mx_quant(int elem, int rceil, int packed, const uint16_t* x, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nblocks = rows * cols / 32;
  if (nblocks == 0) return hipSuccess;
  const int grid = grid_for(nblocks, kMxGridCap);
  const uint4* xv = (const uint4*)x;
  // packed scales need whole 128- or 256-element stages per row, so srow >= 4
  const RowDiv rd = packed ? row_div((uint32_t)(cols / 32)) : RowDiv{(uint32_t)(cols / 32), 0u, 0u};
  if (packed) launch_mx_quant_pks<1>(elem, grid, stream, xv, codes, scales, nblocks, rceil, rd);
  else launch_mx_quant_pks<0>(elem, grid, stream, xv, codes, scales, nblocks, rceil, rd);
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
  const int grid = grid_for(nchunks / 2, kNvGridCap);
  hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(grid), dim3(256), 0, stream, (const uint4*)x, nchunks, codes, scales,
                     tensor_scale, (const uint32_t*)partials, P);
  return hipGetLastError();
}

}  // namespace mxq
