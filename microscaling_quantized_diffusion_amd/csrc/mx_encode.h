// MX block encoding on bf16 bit patterns, shared by the activation quantizer
// and the GEMM epilogue that emits the next layer's quantized activations, so
// that both produce the same codes for the same bf16 values.  Rules: the OCP
// Microscaling Formats v1.0 specification named by the aitrends.kr
// MXFP8/NVFP4 article (Glossary "Microscaling Formats", "MXFP8"): shared
// exponent e = floor(log2(amax)) - emax clamped to [-127, 127] (stored as
// e + 127), elements encoded round-to-nearest-even with saturation, a block
// holding NaN or Inf gets the NaN scale 0xFF and zero codes.  Optional
// round-up rule: e = ceil(log2(amax / max_elem)), the smallest power of two
// that keeps the block maximum within the element range (no saturation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));
typedef short mx_short2 __attribute__((ext_vector_type(2)));
typedef unsigned short mx_ushort2 __attribute__((ext_vector_type(2)));
typedef __bf16 mx_bf16x32 __attribute__((ext_vector_type(32)));
typedef uint32_t mx_u32x16 __attribute__((ext_vector_type(16)));
// Six dwords in registers.  Its in-memory size is padded to 32 bytes: never
// load or store it as a whole, only its elements.
typedef uint32_t mx_u32x6 __attribute__((ext_vector_type(6)));

// emax: exponent of the element format's largest power of two
// (E4M3: 448 = 1.75 * 2^8; E2M1: 6 = 1.5 * 2^2; E2M3: 7.5 = 1.875 * 2^2;
// E3M2: 28 = 1.75 * 2^4).  elem: 1 = E4M3, 2 = E2M1, 3 = E2M3, 4 = E3M2.
template <int ELEM>
constexpr int mx_emax() {
  return ELEM == 1 ? 8 : ELEM == 4 ? 4 : 2;
}

// Largest bf16 magnitude bit pattern of the 4 values in two dwords.  For
// finite values the magnitude order equals the integer order of the bits;
// NaN and Inf compare above every finite value (>= 0x7F80).
__device__ __forceinline__ uint32_t mx_absmax_bits4(uint32_t w0, uint32_t w1) {
  return max(max(w0 & 0x7FFFu, (w0 >> 16) & 0x7FFFu), max(w1 & 0x7FFFu, (w1 >> 16) & 0x7FFFu));
}

// bf16 fraction bits of the element format's largest value's significand
// (448 = 1.75 * 2^8 -> 0x60; 6 = 1.5 * 2^2 -> 0x40; 7.5 = 1.875 * 2^2 ->
// 0x70; 28 = 1.75 * 2^4 -> 0x60).
template <int ELEM>
constexpr uint32_t mx_max_fraction() {
  return ELEM == 1 ? 0x60u : ELEM == 2 ? 0x40u : ELEM == 3 ? 0x70u : 0x60u;
}

// Shared exponent of a finite block from its largest magnitude bit pattern m
// (m < 0x7F80), clamped to [-127, 127]; m == 0 gives -127.
//   rceil == 0: floor(log2(amax)) - emax;
//   rceil == 1: ceil(log2(amax / max_elem)), which is the floor exponent plus
//               one exactly when amax's significand exceeds max_elem's.
template <int ELEM>
__device__ __forceinline__ int mx_shared_exponent(uint32_t m, int rceil) {
  if (m == 0) return -127;
  const int Eb = (int)(m >> 7);
  int fl;
  uint32_t frac;  // 7 fraction bits of amax's significand
  if (Eb) {
    fl = Eb - 127;
    frac = m & 0x7Fu;
  } else {  // subnormal bf16: the top set bit p carries the leading one
    const int p = 31 - __clz(m);
    fl = p - 133;
    frac = (m << (7 - p)) & 0x7Fu;
  }
  const int e = fl - mx_emax<ELEM>() + (rceil & (int)(frac > mx_max_fraction<ELEM>()));
  return min(max(e, -127), 127);
}

__device__ __forceinline__ float mx_pow2f(int e) {  // 2^e for e in [-127, 127], exact
  return e == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(e + 127) << 23);
}

// Four bf16 values (two dwords, element order low half first) -> four E4M3
// codes (one dword, element k in byte k) of x / 2^e.  The gfx950 conversion
// v_cvt_scalef32_pk_fp8_bf16 was measured equal to the RNE-saturating encoding
// wherever |x / 2^e| < 464 (it returns NaN above), so magnitudes are first
// clamped to 448 * 2^e, the value of the largest code 0x7E, which every value
// it replaces also encodes to.
__device__ __forceinline__ uint32_t mx_encode_fp8x4(uint32_t w0, uint32_t w1, int e) {
  const float sc = mx_pow2f(e);
  const unsigned short cap = (unsigned short)(((uint32_t)(e + 135) << 7) | 0x60u);  // 1.75 * 2^(e+8)
  const mx_ushort2 m0 = __builtin_elementwise_min(__builtin_bit_cast(mx_ushort2, w0 & 0x7FFF7FFFu), mx_ushort2{cap, cap});
  const mx_ushort2 m1 = __builtin_elementwise_min(__builtin_bit_cast(mx_ushort2, w1 & 0x7FFF7FFFu), mx_ushort2{cap, cap});
  w0 = __builtin_bit_cast(uint32_t, m0) | (w0 & 0x80008000u);
  w1 = __builtin_bit_cast(uint32_t, m1) | (w1 & 0x80008000u);
  mx_short2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(mx_short2{0, 0}, __builtin_bit_cast(mx_bf16x2, w0), sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(mx_bf16x2, w1), sc, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Four bf16 values -> four E2M1 codes of x / 2^e, written into bytes BYTE and
// BYTE + 1 of `into` (element k in bits 8 BYTE + 4k ..); the other bytes are
// kept.  v_cvt_scalef32_pk_fp4_bf16 was measured equal to the RNE-saturating
// encoding for every finite bf16 and every e in [-127, 127].
template <int BYTE>
__device__ __forceinline__ uint32_t mx_encode_fp4x4(uint32_t into, uint32_t w0, uint32_t w1, int e) {
  static_assert(BYTE == 0 || BYTE == 2, "two bytes per call");
  const float sc = mx_pow2f(e);
  into = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(into, __builtin_bit_cast(mx_bf16x2, w0), sc, BYTE);
  into = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(into, __builtin_bit_cast(mx_bf16x2, w1), sc, BYTE + 1);
  return into;
}

// One 32-element block (four chunks of eight bf16, element order low half
// first) -> its E2M3 (ELEM 3) / E3M2 (ELEM 4) codes of x / 2^e, element j at
// bits 6 j of six dwords.  The gfx950 conversions
// v_cvt_scalef32_pk32_fp6_bf16 / _bf6_bf16 (dividing by the scale operand)
// were measured equal to the RNE-saturating encoding for every finite bf16
// and every e in [-127, 127], with the sign of zero kept.
template <int ELEM>
__device__ __forceinline__ void mx_encode_fp6x32(const uint4 (&v)[4], int e, uint32_t (&out)[6]) {
  static_assert(ELEM == 3 || ELEM == 4, "FP6 element");
  const mx_u32x16 in = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                        v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
  const mx_bf16x32 xv = __builtin_bit_cast(mx_bf16x32, in);
  mx_u32x6 r;
  if constexpr (ELEM == 3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(xv, mx_pow2f(e));
  else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(xv, mx_pow2f(e));
#pragma unroll
  for (int i = 0; i < 6; ++i) out[i] = r[i];
}

}  // namespace mxq
