// Block-scaled FP8 attention for gfx950 (one head dimension: 128).
//
// Method: the devin.kr article on FLUX image generation accelerated on
// Blackwell ("Compute efficiency and acceleration") runs attention in 8-bit
// floating point with a per-token correction of the quantization error.  The
// pages give no steps; this path computes, per head:
//   * Q and K MXFP8-quantized along the head dimension (E4M3 codes, one E8M0
//     scale per 32 channels of each token), V MXFP8-quantized along the token
//     axis (one E8M0 scale per 32 tokens of each channel), the microscaling
//     formats of the aitrends.kr MXFP8/NVFP4 article (Glossary "Microscaling
//     Formats", "MXFP8");
//   * scores from the dequantized codes (scaled MFMA, fp32 accumulate);
//     P = exp(s - m) with m the row's maximum score over all keys, encoded as
//     E4M3 at the fixed scale 2^8; O += P V with V's block scales; the row
//     sum taken over the unquantized P; out = O / l in bf16.  The maximum is
//     exact, not a running one: every P code depends on its own score and m
//     only, whatever order or blocking the keys are visited in.
//
// Kernels
//   vt_quant_kernel   V [S, 128] bf16 -> V^T codes [128, S] and scales
//                     [128, S/32]: a workgroup stages 64 tokens x 128
//                     channels in LDS; each thread encodes one 32-token block
//                     of one channel with the quantizer's block encoding.
//   attn_fp8_kernel   one workgroup = 128 queries of one head (four waves of
//                     32), two passes over the keys, each through two LDS
//                     stages filled by LDS DMA one tile ahead (K rows and V^T
//                     rows XOR-swizzled by 16-byte chunk through the DMA
//                     source offsets, as in the GEMM staging).
//     pass 1          K alone, 128 keys per stage: the scores (the same MFMAs
//                     as pass 2, so the same fp32 values) and their maximum;
//     pass 2          K and V^T, 64 keys per stage (five DMAs per wave), per
//                     tile and wave:
//       S^T = K Q^T    four 32x32x64 scaled MFMAs (K rows are the A operand
//                      from LDS, the wave's 32 queries the B operand, held in
//                      registers for the whole loop);
//       softmax        in the log2 domain with pass 1's maximum: one fused
//                      multiply-add and one exponential per score, no
//                      rescaling; P codes from v_cvt_scalef32_pk_fp8_f32 at
//                      scale 2^-8;
//       P -> operand   the 32x32 accumulator gives lane half h keys 8i + 4h
//                      + (0..3); the MFMA's B operand wants keys 16h .. 16h
//                      + 15 of each 32-key tile, which two permlane32 swaps
//                      per tile produce directly;
//       O^T += V^T P^T four scaled MFMAs (V^T rows from LDS with their E8M0
//                      scales, P with the constant scale 2^-8).
#include "lds_dma.h"
#include "mx_encode.h"
#include "mxq_internal.h"

namespace mxq {
namespace {

typedef int att_v8i __attribute__((ext_vector_type(8)));
typedef float att_v16f __attribute__((ext_vector_type(16)));
typedef float att_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 att_bf16x2 __attribute__((ext_vector_type(2)));
typedef short att_short2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;   // head dimension
constexpr int kBQ = 128;  // queries per workgroup (4 waves x 32)
constexpr int kBK = 64;   // keys per tile
constexpr int kKOff = 0;                       // K tile: 64 rows x 128 code bytes
constexpr int kVOff = kBK * kD;                // V^T tile: 128 rows x 64 code bytes
constexpr int kKsOff = kVOff + kD * kBK;       // K scales: 64 rows x 4 bytes
constexpr int kVsOff = kKsOff + kBK * 4;       // V^T scales: 128 rows x 2 bytes
constexpr int kSinkOff = kVsOff + kD * 2;      // landing area of the two idle scale DMAs
constexpr int kStage = kSinkOff + 512;         // 17408 bytes
constexpr int kPScale = 127 - 8;               // E8M0 byte of 2^-8, the scale of the P codes

__device__ __forceinline__ att_v8i att_as_v8i(const uint4& lo, const uint4& hi) {
  return att_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// v_permlane32_swap(x, y), measured on gfx950: result 0 is x in lanes 0-31
// and y of lane l - 32 in lanes 32-63; result 1 is x of lane l + 32 in lanes
// 0-31 and y in lanes 32-63.  For the P codes of a 32-key accumulator tile
// (dword i of lane half h = keys 8 i + 4 h + 0..3), swap(d0, d2) gives every
// lane its keys 16 h + 0..7 and swap(d1, d3) its keys 16 h + 8..15, in order.
__device__ __forceinline__ void p_regroup(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3, uint32_t* pw) {
  const auto r0 = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
  pw[0] = r0[0];
  pw[1] = r0[1];
  pw[2] = r1[0];
  pw[3] = r1[1];
}
// max / sum of the lane's value and that of lane l ^ 32 (one result of the
// swap is each, in either lane half)
__device__ __forceinline__ float max_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The B operand of S^T for one 32-query block: lane (r32, q) holds its
// query's channels 64 s + 16 q + (0..15) and 64 s + 32 + 16 q + (0..15), and
// the E8M0 scales of channel blocks 2 s + q.
struct QBlock {
  uint4 c[2][2];
  int sc[2];
};
__device__ __forceinline__ QBlock load_qblock(const uint8_t* qc, const uint8_t* qs, size_t row, int q) {
  QBlock b;
  const uint8_t* qp = qc + row * kD;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    b.c[s][0] = *reinterpret_cast<const uint4*>(qp + 64 * s + 16 * q);
    b.c[s][1] = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 + 16 * q);
  }
  const uint32_t w = *reinterpret_cast<const uint32_t*>(qs + row * 4);
  b.sc[0] = (int)((w >> (8 * q)) & 0xFFu);
  b.sc[1] = (int)((w >> (8 * (2 + q))) & 0xFFu);
  return b;
}

// Scores of NT 32-key sub-tiles of a stage against NB 32-query blocks:
// S^T rows krow0 + 32 tt + (0..31) (keys, the A operand from LDS: K rows
// XOR-swizzled by 16-byte chunk, scales 4 bytes per row at kKsOff) x columns
// = queries (the B operand, in registers).  Lane (query r32, half q) gets
// keys krow0 + 32 tt + 8 i + 4 q + (0..3) in elements 4 i + (0..3).  A score
// is the same fp32 value whichever call forms it: the same two MFMAs on the
// same operand bytes, at the same row and column of the product.
template <int NB, int NT>
__device__ __forceinline__ void key_scores(const uint8_t* b, int krow0, const QBlock (&qb)[NB], int r32, int q,
                                           att_v16f (&sacc)[NB][NT]) {
  const int ksw = (r32 >> 1) & 7;  // K row swizzle (invariant under 32-row steps)
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) sacc[j][tt] = att_v16f{};
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int krow = krow0 + 32 * tt + r32;
      const uint8_t* kr = b + kKOff + krow * kD;
      const uint4 a0 = *reinterpret_cast<const uint4*>(kr + (((4 * s + q) ^ ksw) << 4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(kr + (((4 * s + 2 + q) ^ ksw) << 4));
      const int ksc = b[kKsOff + krow * 4 + 2 * s + q];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        sacc[j][tt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            att_as_v8i(a0, a1), att_as_v8i(qb[j].c[s][0], qb[j].c[s][1]), sacc[j][tt], 0, 0, 0, ksc, 0, qb[j].sc[s]);
    }
}

// Four fp32 values in [0, 1] -> four E4M3 codes of p * 2^8 (one dword, value k in byte k).
__device__ __forceinline__ uint32_t p_codes4(float p0, float p1, float p2, float p3) {
  constexpr float kInv = 0x1p-8f;  // the conversion divides by its scale operand
  att_short2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(att_short2{0, 0}, p0, p1, kInv, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, p2, p3, kInv, true);
  return __builtin_bit_cast(uint32_t, r);
}

// V [S, 128] bf16 of head blockIdx.y -> V^T codes [128, S] and scales, the
// scales tile-major ([S/64][128 channels][2 blocks]) so that each 64-key
// tile's 256 scale bytes are contiguous for the attention kernel's DMA.
// Workgroup: tokens 64 * blockIdx.x .. + 63; thread t: channel t % 128, 32-token block t / 128.
__global__ __launch_bounds__(256) void vt_quant_kernel(const uint16_t* __restrict__ v, uint8_t* __restrict__ vt_codes,
                                                       uint8_t* __restrict__ vt_scales, int S) {
  constexpr int kPitch = kD + 2;  // u16 per LDS row: a 4-byte pad keeps column reads spread over banks
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kPitch];
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const uint16_t* src = v + ((size_t)bh * S + t0) * kD;
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // 64 rows x 16 chunks of 16 bytes
    const int g = threadIdx.x + 256 * u;
    const int row = g >> 4, col = (g & 15) * 8;
    const uint4 val = *reinterpret_cast<const uint4*>(src + (size_t)row * kD + col);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * kPitch + col);
    dst[0] = val.x;
    dst[1] = val.y;
    dst[2] = val.z;
    dst[3] = val.w;
  }
  __syncthreads();
  const int c = threadIdx.x & (kD - 1), blk = threadIdx.x >> 7;
  uint32_t w[16];  // tokens 32 blk + 2j (low half) and + 2j + 1 (high half) of channel c
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t lo = tile[(32 * blk + 2 * j) * kPitch + c];
    const uint32_t hi = tile[(32 * blk + 2 * j + 1) * kPitch + c];
    w[j] = lo | (hi << 16);
    m = max(m, max(lo & 0x7FFFu, hi & 0x7FFFu));
  }
  uint32_t code[8];
  uint32_t sbyte;
  if (m >= 0x7F80u) {  // NaN or Inf in the block: NaN scale, zero codes
    sbyte = 0xFFu;
#pragma unroll
    for (int k = 0; k < 8; ++k) code[k] = 0;
  } else {
    const int e = mx_shared_exponent<1>(m, 0);
    sbyte = (uint32_t)(e + 127);
#pragma unroll
    for (int k = 0; k < 8; ++k) code[k] = mx_encode_fp8x4(w[2 * k], w[2 * k + 1], e);
  }
  uint8_t* dst = vt_codes + ((size_t)bh * kD + c) * S + t0 + 32 * blk;
  *reinterpret_cast<uint4*>(dst) = make_uint4(code[0], code[1], code[2], code[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(code[4], code[5], code[6], code[7]);
  vt_scales[((size_t)bh * (S / 64) + blockIdx.x) * (2 * kD) + 2 * c + blk] = (uint8_t)sbyte;
}

// Attention of 128 queries of head blockIdx.y.  Q, K: codes [BH*S, 128] and
// scales [BH*S, 4]; V^T: codes [BH*128, S] and tile-major scales
// [BH][S/64][128][2].  S is a multiple of 64; c_log2 = log2(e) / sqrt(128).
// Output: REQ 0: bf16 [BH*S, 128] in `out`.  REQ 1 / 2: MX-quantized (E4M3 /
// E2M1 codes, E8M0 scales per 32 channels, rceil selecting the round-up rule)
// token-major, heads side by side: row b*S + s, columns h*128 + d, rows qld
// code bytes and sld scale bytes apart; the bf16 values quantized are those
// REQ 0 would store.
template <int REQ>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(const uint8_t* __restrict__ qc,
                                                          const uint8_t* __restrict__ qs,
                                                          const uint8_t* __restrict__ kc,
                                                          const uint8_t* __restrict__ ks,
                                                          const uint8_t* __restrict__ vtc,
                                                          const uint8_t* __restrict__ vts,
                                                          uint16_t* __restrict__ out, int S, float c_log2,
                                                          uint8_t* __restrict__ qcodes,
                                                          uint8_t* __restrict__ qscales, int64_t qld, int64_t sld,
                                                          int H, int rceil) {
  // one __shared__ array per stage, each named at compile time in the
  // unrolled loop, so the compiler waits only on the stage being read
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 5, r32 = lane & 31;
  const int bh = blockIdx.y;
  const int qrow = blockIdx.x * kBQ + wave * 32 + r32;
  const bool qvalid = qrow < S;
  const int qr = qvalid ? qrow : S - 1;  // rows past S compute on a valid row and store nothing

  // B operand of S^T in pass 2: this wave's 32 queries
  const QBlock qa[1] = {load_qblock(qc, qs, (size_t)bh * S + qr, q)};

  // DMA sources: this head's K codes, K scales, V^T codes and V^T scales
  const uint32_t head_bytes = (uint32_t)S * kD;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + (size_t)bh * head_bytes, head_bytes);
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(ks + (size_t)bh * S * 4, (uint32_t)S * 4);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vtc + (size_t)bh * head_bytes, head_bytes);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(vts + (size_t)bh * (S / 64) * (2 * kD), (uint32_t)(S / 64) * (2 * kD));
  // Per-lane source offsets without the tile term.  A wave-wide 16-byte DMA
  // fills 1 KiB of LDS in lane order: K rows 8 g .. 8 g + 7 of the tile
  // (chunk g), V^T rows 16 g .. 16 g + 15; each lane fetches the chunk whose
  // swizzled position is its own.  K row 8 g + x has swizzle ((8 g + x) >> 1)
  // & 7 = (4 (g & 1) + (x >> 1)) & 7, so two per-lane K offsets serve every
  // chunk (kbase[g & 1]; the row term 8 g * 128 goes into the wave-uniform
  // offset).  Pass 2 scales: wave 0 the tile's K scales, wave 1 its V^T
  // scales (256 bytes each), waves 2 and 3 nothing (out of range, into the sink).
  uint32_t kbase[2], voff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int x = lane >> 3, kp = lane & 7;
    kbase[u] = (uint32_t)x * kD + (uint32_t)((kp ^ ((4 * u + (x >> 1)) & 7)) << 4);
    const int g = 2 * wave + u;
    const int vr = 16 * g + (lane >> 2), vp = lane & 3;
    voff[u] = (uint32_t)vr * (uint32_t)S + (uint32_t)((vp ^ ((vr >> 2) & 3)) << 4);
  }
  const uint32_t soff = wave < 2 ? (uint32_t)lane * 4 : kOutOfRange;
  const __amdgpu_buffer_rsrc_t rsc = wave == 1 ? rvs : rks;
  const int ntiles = S / kBK;
  // Pass-2 stage j holds K of tile j and V^T of tile j - 1 with their scales
  // (tile t of either scale array starts at byte 256 t).  A missing tile (K
  // past the last, V before the first) reads a zero-length range: zeros.
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(kc, 0u);
  auto issue = [&](auto& st, int j) {
    const bool hk = j < ntiles, hv = j >= 1 && j - 1 < ntiles;
    const __amdgpu_buffer_rsrc_t rkj = hk ? rk : rnone, rvj = hv ? rv : rnone;
    const uint32_t ko = hk ? (uint32_t)j * kBK * kD : 0u, vo = hv ? (uint32_t)(j - 1) * kBK : 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      lds_dma16(rkj, &st[kKOff + 1024 * (2 * wave + u)], kbase[u], ko + (uint32_t)(8 * (2 * wave + u)) * kD);
      lds_dma16(rvj, &st[kVOff + 1024 * (2 * wave + u)], voff[u], vo);
    }
    const bool hs = wave == 1 ? hv : hk;
    lds_dma4(hs ? rsc : rnone, &st[kKsOff + 256 * wave], soff, hs ? (wave == 1 ? vo : ko / kD) * 4u : 0u);
  };

  // Pass 1: the row maximum of the raw scores over all keys.  A stage holds
  // 128 K rows (16 KiB over its K and V^T areas; chunk g = 4 wave + u) and
  // their 512 scale bytes at kKsOff (waves 0 and 1); the tile after the last
  // one is not loaded.  Wave w takes queries 64 (w & 1) + (0..63) of the
  // workgroup (two 32-query blocks) against keys 64 (w >> 1) + (0..63) of
  // each stage: eight MFMAs per stage and wave, as with 32 queries against
  // all 128 keys, on half the LDS reads.  S is a multiple of 64, so a last
  // stage past S holds 64 keys (the rest loads as zeros and is not read), all
  // in the first key half.
  auto issue_k = [&](auto& st, int kv0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = 4 * wave + u;
      lds_dma16(rk, &st[kKOff + 1024 * g], kbase[u & 1], (uint32_t)(kv0 + 8 * g) * kD);
    }
    if (wave < 2) lds_dma4(rks, &st[kKsOff + 256 * wave], (uint32_t)lane * 4, (uint32_t)(kv0 + 64 * wave) * 4);
  };
  const int qhalf = wave & 1, khalf = wave >> 1;
  QBlock qm[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = blockIdx.x * kBQ + 64 * qhalf + 32 * j + r32;
    qm[j] = load_qblock(qc, qs, (size_t)bh * S + (row < S ? row : S - 1), q);
  }
  const int n1 = (S + 127) / 128;
  float mx[2] = {-INFINITY, -INFINITY};
  auto mstep = [&](auto& cur, auto& nxt, int t) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (t + 1 < n1) issue_k(nxt, (t + 1) * 128);
    if (128 * t + 64 * khalf < S) {
      att_v16f sacc[2][2];
      key_scores<2, 2>(cur, 64 * khalf, qm, r32, q, sacc);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx[j] = fmaxf(mx[j], sacc[j][tt][r]);
    }
  };
  issue_k(st0, 0);
  int t = 0;
  for (; t + 1 < n1; t += 2) {
    mstep(st0, st1, t);
    mstep(st1, st0, t + 1);
  }
  if (t < n1) mstep(st0, st1, t);
  // the two key halves' maxima of every query meet in LDS
  __shared__ float mpart[2][kBQ];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float v = max_half(mx[j]);
    if (q == 0) mpart[khalf][64 * qhalf + 32 * j + r32] = v;
  }
  __builtin_amdgcn_s_barrier();  // every wave has read its last pass-1 stage and written its maxima
  // p = exp2(s c_log2 - m): the maximum is taken over the raw scores (the
  // scale c_log2 is positive), so the largest p is 1 up to the rounding of m
  const float m = fmaxf(mpart[0][32 * wave + r32], mpart[1][32 * wave + r32]) * c_log2;

  att_v16f acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = att_v16f{};
  float l = 0.0f;
  const int vsw = (r32 >> 2) & 3;  // V^T row swizzle

  // P codes of one tile's scores (p = exp2(s c_log2 - m), with the row sum of
  // the unquantized p added to l), then O^T += V^T P^T with V^T from `b`
  auto softmax_pv = [&](const uint8_t* b, const att_v16f (&sc)[1][2]) {
    float ls = 0.0f;
    uint32_t d[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][tt][4 * i + u], c_log2, -m));
          ls += p[u];
        }
        d[tt][i] = p_codes4(p[0], p[1], p[2], p[3]);
      }
    l += ls;

    // P codes into the B-operand layout: lane half q holds keys 16 q .. 16 q + 15 of each tile
    uint32_t pw[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) p_regroup(d[tt][0], d[tt][1], d[tt][2], d[tt][3], pw + 4 * tt);
    const att_v8i pop = att_v8i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                                (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};

    // O^T += V^T P^T: channels 32 c + (0..31) x the wave's 32 queries
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int vrow = 32 * c + r32;
      const uint8_t* vr = b + kVOff + vrow * kBK;
      const uint4 a0 = *reinterpret_cast<const uint4*>(vr + ((q ^ vsw) << 4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(vr + (((2 + q) ^ vsw) << 4));
      const int vsc = b[kVsOff + vrow * 2 + q];
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(att_as_v8i(a0, a1), pop, acc[c], 0, 0, 0, vsc, 0,
                                                               kPScale);
    }
  };

  // Pass 2, step j (1 <= j <= ntiles): stage j has landed in `cur` (own wait,
  // then the barrier for everyone's); stage j + 1 goes into `nxt`, which every
  // wave has finished reading.  The scores of tile j (MFMAs; zeros for
  // j = ntiles, unused) are issued first, so that the matrix cores form them
  // while the VALU turns the previous tile's scores into P codes; then P V of
  // tile j - 1.
  auto step = [&](auto& cur, auto& nxt, int j, att_v16f (&snew)[1][2], const att_v16f (&sold)[1][2]) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    issue(nxt, j + 1);
    key_scores<1, 2>(cur, 0, qa, r32, q, snew);
    softmax_pv(cur, sold);
  };

  att_v16f sa[1][2], sb[1][2];
  issue(st0, 0);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  issue(st1, 1);
  key_scores<1, 2>(st0, 0, qa, r32, q, sa);  // scores of tile 0
  int j = 1;
  for (; j + 1 <= ntiles; j += 2) {
    step(st1, st0, j, sb, sa);
    step(st0, st1, j + 1, sa, sb);
  }
  if (j == ntiles) step(st1, st0, j, sb, sa);
  wait_vmcnt<0>();  // the last (empty) DMA lands before the workgroup's LDS is released

  // out = O / l: lane (query, q) holds channels 32 c + 8 i + 4 q + (0..3)
  const float inv = 1.0f / sum_half(l);
  if constexpr (REQ == 0) {
    if (qvalid) {
      uint16_t* orow = out + ((size_t)bh * S + qrow) * kD;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const att_bf16x2 lo = __builtin_convertvector(att_f32x2{acc[c][4 * i] * inv, acc[c][4 * i + 1] * inv},
                                                        att_bf16x2);
          const att_bf16x2 hi = __builtin_convertvector(
              att_f32x2{acc[c][4 * i + 2] * inv, acc[c][4 * i + 3] * inv}, att_bf16x2);
          *reinterpret_cast<uint2*>(orow + 32 * c + 8 * i + 4 * q) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
    }
  } else {
    // The same bf16 values, MX-quantized per 32 channels: a block is this
    // lane's 16 values and the other lane half's 16 (the amax is exchanged
    // with one swap); codes and scale as the standalone quantizer makes them.
    const int b = bh / H, h = bh % H;
    const size_t orow = (size_t)b * S + qrow;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t w[8];  // bf16 pairs: channels 8 i + 4 q + (0, 1) and (2, 3)
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const att_bf16x2 lo = __builtin_convertvector(att_f32x2{acc[c][4 * i] * inv, acc[c][4 * i + 1] * inv},
                                                      att_bf16x2);
        const att_bf16x2 hi = __builtin_convertvector(att_f32x2{acc[c][4 * i + 2] * inv, acc[c][4 * i + 3] * inv},
                                                      att_bf16x2);
        w[2 * i] = __builtin_bit_cast(uint32_t, lo);
        w[2 * i + 1] = __builtin_bit_cast(uint32_t, hi);
        m = max(m, mx_absmax_bits4(w[2 * i], w[2 * i + 1]));
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(m, m, false, false);
      m = max(sw[0], sw[1]);
      const bool nonfinite = m >= 0x7F80u;  // NaN or Inf in the block: NaN scale, zero codes
      const int e = nonfinite ? 0 : mx_shared_exponent<REQ>(m, rceil);
      if (qvalid) {
        const int col = h * kD + 32 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = col + 8 * i + 4 * q;
          if constexpr (REQ == 1) {
            const uint32_t code = nonfinite ? 0u : mx_encode_fp8x4(w[2 * i], w[2 * i + 1], e);
            *reinterpret_cast<uint32_t*>(qcodes + orow * (size_t)qld + ch) = code;
          } else {
            const uint32_t code = nonfinite ? 0u : mx_encode_fp4x4<0>(0u, w[2 * i], w[2 * i + 1], e);
            *reinterpret_cast<uint16_t*>(qcodes + orow * (size_t)qld + ch / 2) = (uint16_t)code;
          }
        }
        if (q == 0) qscales[orow * (size_t)sld + col / 32] = nonfinite ? 0xFFu : (uint8_t)(e + 127);
      }
    }
  }
}

}  // namespace

AttentionLayout attention_layout(int64_t BH, int64_t S) {
  auto r256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  AttentionLayout L{};
  const size_t codes = (size_t)BH * (size_t)S * kD, scales = codes / 32;
  L.q_codes = 0;
  L.q_scales = L.q_codes + r256(codes);
  L.k_codes = L.q_scales + r256(scales);
  L.k_scales = L.k_codes + r256(codes);
  L.vt_codes = L.k_scales + r256(scales);
  L.vt_scales = L.vt_codes + r256(codes);
  L.total = L.vt_scales + r256(scales);
  return L;
}

hipError_t launch_attention_fp8(int64_t BH, int64_t S, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* out, uint8_t* ws, hipStream_t stream, int out_elem, int rceil, int64_t H,
                                uint8_t* qcodes, uint8_t* qscales, int64_t qld, int64_t sld) {
  const AttentionLayout L = attention_layout(BH, S);
  hipError_t e = launch_mx_quant(1, 0, 0, q, BH * S, kD, ws + L.q_codes, ws + L.q_scales, stream);
  if (e != hipSuccess) return e;
  e = launch_mx_quant(1, 0, 0, k, BH * S, kD, ws + L.k_codes, ws + L.k_scales, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vt_quant_kernel, dim3((unsigned)(S / 64), (unsigned)BH), dim3(256), 0, stream, v,
                     ws + L.vt_codes, ws + L.vt_scales, (int)S);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c_log2 = 1.4426950408889634f / 11.313708498984761f;  // log2(e) / sqrt(128)
  const dim3 grid((unsigned)((S + kBQ - 1) / kBQ), (unsigned)BH);
  if (out_elem == 0)
    hipLaunchKernelGGL(attn_fp8_kernel<0>, grid, dim3(256), 0, stream, ws + L.q_codes, ws + L.q_scales,
                       ws + L.k_codes, ws + L.k_scales, ws + L.vt_codes, ws + L.vt_scales, out, (int)S, c_log2,
                       nullptr, nullptr, (int64_t)0, (int64_t)0, (int)H, 0);
  else if (out_elem == 1)
    hipLaunchKernelGGL(attn_fp8_kernel<1>, grid, dim3(256), 0, stream, ws + L.q_codes, ws + L.q_scales,
                       ws + L.k_codes, ws + L.k_scales, ws + L.vt_codes, ws + L.vt_scales, nullptr, (int)S, c_log2,
                       qcodes, qscales, qld, sld, (int)H, rceil);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<2>, grid, dim3(256), 0, stream, ws + L.q_codes, ws + L.q_scales,
                       ws + L.k_codes, ws + L.k_scales, ws + L.vt_codes, ws + L.vt_scales, nullptr, (int)S, c_log2,
                       qcodes, qscales, qld, sld, (int)H, rceil);
  return hipGetLastError();
}

}  // namespace mxq
