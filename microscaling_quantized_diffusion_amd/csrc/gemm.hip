// GEMMs on the gfx950 matrix cores for the block-scaled formats and bf16,
// computing out[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k] (+ bias[n]) with an
// fp32 accumulator and a nearest-even bf16 result.  This is the GEMM of the
// aitrends.kr MXFP8/NVFP4 article ("Section details": quantized weights times
// dynamically quantized activations; second "Evidence" block: small layers
// stay in bf16).  Kernels:
//   mxe_gemm_kernel   (gemm_mx_kernel.h) the MX main path: whole-stage
//                     MXFP8 / MXFP6 / MXFP4 GEMMs on 256x256, 256x320 or
//                     384x192 tiles, scaled 32x32x64 MFMA (hardware E8M0 block
//                     scales), two-stage LDS-DMA ring of 128-byte K slabs,
//                     stages published early; with a bf16 epilogue
//                     (gemm_mx.hip) or one that quantizes its output for the
//                     next layer (gemm_mx_requant.hip).
//   mxp_gemm_kernel   the same tiles and ring with the stage published at its
//                     start: MXFP4 on 256x320 tiles (the early-published
//                     kernel's registers do not fit them).
//   nv4_gemm_kernel   NVFP4 main path: the same tile and ring; codes widened
//                     to f16 with the E4M3 block scale applied (exact), f16
//                     32x32x16 MFMA, tensor scales in the epilogue.
//   gemm_kernel       generic 16x16 path for every mode (MX8 / MX4 / NV4 /
//                     BF16) and shape: K not a multiple of the main paths'
//                     slab, unaligned scale rows, and the bf16 MFMA GEMM.
//   bf16_skinny_kernel / bf16_generic_kernel   bf16 fallback for up to 16
//                     activation rows (an HBM stream of W) and for K % 8 != 0.
// Weights are the MFMA "A" operand and activations the "B" operand, so a
// lane's accumulators are consecutive output columns of one output row.
// Every kernel's buffer resources span only the tile's rows, so rows past
// M / N and the K tail read as zeros.
#include <utility>

#include "gemm_tile.h"

namespace mxq {
namespace {

enum Mode { MX8 = 1, MX4 = 2, NV4 = 3, BF16 = 4 };

template <int FMT, int OPA, int OPB>
__device__ __forceinline__ v4f mfma_scaled(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, OPA, sa, OPB, sb);
}

// XOR swizzles of the 16-byte chunk index by row, chosen by measurement on
// gfx950 (SQ_LDS_BANK_CONFLICT = 0 for the operand read pattern):
//   swz  : 16 consecutive rows read the same logical chunk (16x16 operands)
__device__ __forceinline__ int swz(int r) { return r & 7; }

__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xF, m = c & 7;
  // E4M3 (bias 7) is a subset of f16 (bias 15): normal -> exponent + 8;
  // subnormal m * 2^-9 -> exact f16 normal/subnormal via integer convert.
  if (e == 0) return (_Float16)((float)m * 0x1p-9f);
  const uint16_t bits = (uint16_t)(((e + 8u) << 10) | (m << 7));
  return __builtin_bit_cast(_Float16, bits);
}

// 8 NVFP4 codes (one dword) -> 8 f16 values times the block scale.
__device__ __forceinline__ void nv4_dequant_dword(uint32_t x, h2 s2, h2 (&o)[4]) {
  o[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s2;
  o[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s2;
  o[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2;
  o[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s2;
}

// Generic path.  Data flow per workgroup (one BM x BN output tile):
//   global --buffer_load_dwordx4 ... lds (LDS DMA, no VGPR staging)--> LDS
//   (two stages; every row holds one 128-byte K slab; 16-byte chunks are
//   XOR-swizzled by row) --ds_read_b128--> MFMA operands.  The loads of K
//   step k+1 are in flight while step k computes.  Per-lane scale bytes are
//   read from global memory one K step ahead.
// Operand layouts (measured on gfx950):
//   scaled 16x16x128: lane l serves row l % 16 and K-quarter q = l / 16;
//     FP8 operand bytes 0-15 = K [16q, 16q+16), bytes 16-31 = K [64+16q, +16);
//     FP4 operand bytes 0-15 = K [32q, 32q+32), low nibble first;
//     the scale byte of lane l is that of K-block q of row l % 16.
//   bf16/f16 16x16x32: lane l holds 8 K-values of row l % 16; any K order
//     works as long as both operands use the same one.
// Every mode therefore reads 16-byte chunks q and 4+q of each 128-byte row
// slab, and the accumulators of lane l are 4 consecutive output columns of
// one output row (8-byte stores in the epilogue).  NV4 codes (one dword = 8
// elements inside one 16-element block) are widened with
// v_cvt_scalef32_pk_f16_fp4 at unit scale and multiplied by the E4M3 block
// scale with v_pk_mul_f16 (e2m1 * e4m3 needs at most 6 significant bits and
// lies in [2^-10, 2688]: exact in f16); the tensor scales multiply the fp32
// result.
template <int MODE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ Ws, const float* __restrict__ a_ts, const float* __restrict__ w_ts,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int N, int K) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TJ = WTM / 16, TI = WTN / 16;  // 16x16 MFMA tiles per wave (M, N)
  constexpr int ROWS = BM + BN;                // LDS rows per stage (A rows, then W rows)
  constexpr int GROUPS = ROWS / 8;             // 8-row (1 KiB) groups, one wave-wide load each
  static_assert(BM % 16 == 0 && BN % 16 == 0 && GROUPS % NW == 0, "tile/wave mismatch");
  constexpr int PER_WAVE = GROUPS / NW;
  // scale bytes per lane per K step and row: MX8 1, MX4 2 (E8M0); NV4 4 (E4M3)
  constexpr int NSC = (MODE == MX8) ? 1 : (MODE == MX4) ? 2 : (MODE == NV4) ? 4 : 0;
  constexpr int NSC1 = NSC > 0 ? NSC : 1;
  constexpr int FMT = (MODE == MX8) ? 0 : 4;  // cbsz / blgp: 0 = FP8 E4M3, 4 = FP4 E2M1

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // 2 stages x ROWS x 128 bytes

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 4, r16 = lane & 15;

  // tile assignment: XCD-contiguous ids, then groups of 8 M-tiles sweeping N
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  constexpr int GROUP = 8;
  const int group = (int)(id / (uint32_t)(GROUP * tiles_n));
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (int)(id % (uint32_t)gsz);
  const int tn = (int)((id % (uint32_t)(GROUP * tiles_n)) / (uint32_t)gsz);
  const int m0 = tm * BM, n0 = tn * BN;

  const int KB = (MODE == MX8) ? K : (MODE == BF16) ? 2 * K : K / 2;  // bytes per row
  const int SK = (MODE == NV4) ? K / 16 : K / 32;                     // scale bytes per row
  const int nk = (KB + 127) / 128;                                    // K steps

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * KB, (uint32_t)min(BM, M - m0) * (uint32_t)KB);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * KB, (uint32_t)min(BN, N - n0) * (uint32_t)KB);

  // ---- global -> LDS without VGPR staging: each lane moves one 16-byte chunk.
  // LDS row r of group g holds chunk (lane & 7) at physical slot (lane & 7),
  // i.e. logical chunk (lane & 7) ^ swz(r) of the tile row.
  auto issue_stage = [&](int ks, int stage) {
    uint8_t* sbase = smem + stage * (ROWS * 128);
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int g = wave * PER_WAVE + u;
      const int r = g * 8 + (lane >> 3);
      const bool isA = g * 8 < BM;
      const int rr = isA ? r : r - BM;
      const int kb = ks * 128 + (((lane & 7) ^ swz(r)) << 4);
      const uint32_t off = kb < KB ? (uint32_t)rr * (uint32_t)KB + (uint32_t)kb : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rw, &sbase[g * 1024], 16, off, 0, 0, 0);
    }
  };

  // ---- per-lane scale bytes of one K step, four per VGPR.
  // MX: slot h -> K-block 4*NSC*ks + 4h + q.
  // NV4: slots {2q, 2q+1, 8+2q, 9+2q} of the step's 16 blocks (chunk q and 4+q).
  // Slot (t, h) of tile t lives in byte (t*NSC + h) % 4 of word (t*NSC + h) / 4.
  constexpr int SWW = (TI * NSC1 + 3) / 4, SWA = (TJ * NSC1 + 3) / 4;
  auto scale_block = [&](int ks, int h) -> int {
    if (MODE == NV4) return ks * 16 + (h >> 1) * 8 + 2 * q + (h & 1);
    return ks * (4 * NSC) + 4 * h + q;
  };
  uint32_t scW[SWW], scA[SWA];
  auto load_scales = [&](int ks, uint32_t (&sw)[SWW], uint32_t (&sa)[SWA]) {
#pragma unroll
    for (int w = 0; w < SWW; ++w) sw[w] = 0;
#pragma unroll
    for (int w = 0; w < SWA; ++w) sa[w] = 0;
    if (NSC == 0) return;
#pragma unroll
    for (int h = 0; h < NSC; ++h) {
      const int kblk = scale_block(ks, h);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int n = n0 + wn * WTN + 16 * i + r16;
        const uint32_t b = (n < N && kblk < SK) ? (uint32_t)Ws[(size_t)n * SK + kblk] : 0u;
        const int L = i * NSC + h;
        sw[L / 4] |= b << (8 * (L % 4));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int m = m0 + wm * WTM + 16 * j + r16;
        const uint32_t b = (m < M && kblk < SK) ? (uint32_t)As[(size_t)m * SK + kblk] : 0u;
        const int L = j * NSC + h;
        sa[L / 4] |= b << (8 * (L % 4));
      }
    }
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue_stage(0, 0);
  load_scales(0, scW, scA);

  for (int ks = 0; ks < nk; ++ks) {
    // stage ks&1 has landed for every wave, and every wave is done reading
    // stage (ks+1)&1 from the previous step
    wait_vmcnt<0>();
    __syncthreads();
    const bool more = ks + 1 < nk;
    if (more) issue_stage(ks + 1, (ks + 1) & 1);
    uint32_t nscW[SWW], nscA[SWA];
    if (more) load_scales(ks + 1, nscW, nscA);

    const uint8_t* sA = smem + (ks & 1) * (ROWS * 128);
    const uint8_t* sW = sA + BM * 128;
    uint4 fa[TJ][2];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = wm * WTM + 16 * j + r16;
      const uint8_t* base = sA + row * 128;
      fa[j][0] = *reinterpret_cast<const uint4*>(base + ((q ^ swz(row)) << 4));
      fa[j][1] = *reinterpret_cast<const uint4*>(base + (((4 + q) ^ swz(row)) << 4));
    }
    static_for<TI>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      uint4 fw[2];
      {
        const int row = wn * WTN + 16 * i + r16;
        const uint8_t* base = sW + row * 128;
        fw[0] = *reinterpret_cast<const uint4*>(base + ((q ^ swz(row)) << 4));
        fw[1] = *reinterpret_cast<const uint4*>(base + (((4 + q) ^ swz(row)) << 4));
      }
      if constexpr (MODE == MX8) {
        constexpr int LW = i;
        static_for<TJ>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          acc[i][j] = mfma_scaled<FMT, LW % 4, j % 4>(as_v8i(fw[0], fw[1]), as_v8i(fa[j][0], fa[j][1]), acc[i][j],
                                                      (int)scW[LW / 4], (int)scA[j / 4]);
        });
      } else if constexpr (MODE == MX4) {
        static_for<2>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          constexpr int LW = i * 2 + h;
          static_for<TJ>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int LA = j * 2 + h;
            acc[i][j] = mfma_scaled<FMT, LW % 4, LA % 4>(as_v8i_lo(fw[h]), as_v8i_lo(fa[j][h]), acc[i][j],
                                                         (int)scW[LW / 4], (int)scA[LA / 4]);
          });
        });
      } else if constexpr (MODE == BF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, fw[h]),
                                                                 __builtin_bit_cast(v8bf, fa[j][h]), acc[i][j], 0, 0,
                                                                 0);
      } else {  // NV4: 8 f16 MFMAs per step, one per dword d of (chunk q | chunk 4+q)
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const int half = d >> 2, dw = d & 3;
          const int slot = half * 2 + (dw >> 1);  // 16-element block of this dword
          const uint32_t xw = (dw == 0) ? fw[half].x : (dw == 1) ? fw[half].y : (dw == 2) ? fw[half].z : fw[half].w;
          const int LW = i * 4 + slot;
          const _Float16 sw16 = e4m3_to_f16((scW[LW / 4] >> (8 * (LW % 4))) & 0xFFu);
          h2 ow[4];
          nv4_dequant_dword(xw, h2{sw16, sw16}, ow);
          const v8h wa = v8h{ow[0].x, ow[0].y, ow[1].x, ow[1].y, ow[2].x, ow[2].y, ow[3].x, ow[3].y};
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
            const uint32_t xa = (dw == 0) ? fa[j][half].x : (dw == 1) ? fa[j][half].y : (dw == 2) ? fa[j][half].z
                                                                                               : fa[j][half].w;
            const int LA = j * 4 + slot;
            const _Float16 sa16 = e4m3_to_f16((scA[LA / 4] >> (8 * (LA % 4))) & 0xFFu);
            h2 oa[4];
            nv4_dequant_dword(xa, h2{sa16, sa16}, oa);
            const v8h ab = v8h{oa[0].x, oa[0].y, oa[1].x, oa[1].y, oa[2].x, oa[2].y, oa[3].x, oa[3].y};
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, ab, acc[i][j], 0, 0, 0);
          }
        }
      }
    });

    if (more) {
#pragma unroll
      for (int w = 0; w < SWW; ++w) scW[w] = nscW[w];
#pragma unroll
      for (int w = 0; w < SWA; ++w) scA[w] = nscA[w];
    }
  }

  // ---- epilogue: (x tensor scales) (+ bias) -> bf16 RNE -> global
  float alpha = 1.0f;
  if (MODE == NV4) alpha = a_ts[0] * w_ts[0];
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int n = n0 + wn * WTN + 16 * i + 4 * q;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
#pragma unroll
      for (int v = 0; v < 4; ++v) bv[v] = (n + v < N) ? bf16_to_f32(bias[n + v]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int m = m0 + wm * WTM + 16 * j + r16;
      if (m >= M) continue;
      uint32_t h[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float y = (MODE == NV4) ? acc[i][j][v] * alpha : acc[i][j][v];
        h[v] = f32_to_bf16_rne(y + bv[v]);
      }
      uint16_t* dst = out + (size_t)m * N + n;
      if (vec_ok && n + 3 < N) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + v < N) dst[v] = (uint16_t)h[v];
      }
    }
  }
}

template <int MODE, int BM, int BN, int WM, int WN>
hipError_t launch_tiled(int64_t M, int64_t N, int64_t K, const void* a, const uint8_t* as, const void* w,
                        const uint8_t* ws, const float* a_ts, const float* w_ts, const uint16_t* bias, uint16_t* out,
                        hipStream_t stream) {
  constexpr size_t lds = 2 * (size_t)(BM + BN) * 128;
  auto kern = gemm_kernel<MODE, BM, BN, WM, WN>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(64 * WM * WN), lds, stream, (const uint8_t*)a, as,
                     (const uint8_t*)w, ws, a_ts, w_ts, bias, out, (int)M, (int)N, (int)K);
  return hipGetLastError();
}


// ------------------------------------------------------------------------
// MX main path.  One BM x BN output tile per workgroup (default 256 x 256,
// eight waves as 4 x 2, each 64 x 128 outputs in fp32 accumulators), 32x32x64
// scaled MFMA, and an NS-stage LDS ring of SLAB-byte K slabs (SLAB = 128:
// 128 FP8 / FP6 or 256 FP4 elements per row; SLAB = 64: half that) filled by
// LDS DMA NS-1 stages ahead of use.  An FP6 row stores each 32-element block
// in a 32-byte slot (24 code bytes, 8 zero bytes), so it stages exactly like
// an FP8 row.
//
// * Staging.  Measured on gfx950, L2 -> LDS DMA throughput tracks the
//   contiguous bytes each instruction reads per row (32 B: 8, 64 B: 16,
//   128 B: 29 TB/s), and a 256 x 256 tile needs 128 MACs per staged byte.
//   Each stage lives in its own __shared__ array and the loop is unrolled by
//   NS, so that every array is named at compile time: the compiler then
//   tracks the DMA per array and never waits on a stage other than the one
//   being read.  The per-lane source offset is a loop-invariant register and
//   the K step goes into the instruction's scalar offset (a temporary offset
//   register, once reused, makes the compiler wait for the DMA).  Cross-wave
//   visibility: wait for the wave's own DMA (vmcnt through the builtin, which
//   the compiler's bookkeeping sees), then s_barrier.
// * Scales ride with the codes of each stage: per row one dword of E8M0
//   bytes (FP8 / FP6: K-blocks 4p .. 4p+3 of the stage's 128 K-elements;
//   FP4: SLAB/64 dwords).
// * LDS layout.  Row r's SLAB bytes at r * SLAB, its 16-byte chunks
//   XOR-swizzled by (r >> 1) & 7 (128-byte rows) or (r >> 2) & 3 (64-byte
//   rows), both measured conflict-free for the operand reads.
// * Operands.  Lane (r, q) of a 32x32x64 MFMA holds 16-byte chunks 4h + q
//   and 4h + 2 + q of row r for the 64-byte half h of a slab (FP8, FP4), or
//   chunks 4h + 2q and 4h + 2q + 1, the slot of K-block q, whose six code
//   dwords the FP6 MFMA reads and whose two zero dwords it ignores.  Each wave
//   streams its W tiles through two register slots, the reads of the next
//   MFMA group issued ahead of the current one (see stream_stage).  Lane q's
//   scale is that of K-block q of the MFMA's 64 K-elements: FP8 / FP6 block
//   2h + q of the stage, FP4 blocks 4h + q and 4h + 2 + q for its two MFMAs.
// * Measured on gfx950 (s_memtime per wave and stage, FLUX MLP up-projection):
//   the DMA wait before the stage barrier is ~1% of the loop; the barrier
//   ~20%, because the older wave of each SIMD wins issue and finishes its
//   MFMAs first, and the younger one then runs alone on LDS latency.  Wave
//   priorities (s_setprio around MFMA groups), deeper read pipelines, an L2
//   prefetch of the next K slab and fewer scale DMAs all left the time
//   unchanged.  The operand reads use about a third of the LDS's measured
//   256 B/clk read bandwidth at full MFMA rate, so the loop is bound by LDS
//   latency and the per-stage barrier, not by LDS bytes.
// * Epilogue.  (+ bias) -> bf16 RNE; each wave stages 32 output rows at a
//   time through the idle stage buffers (16-byte row pad) and writes whole
//   256-byte row segments with 16-byte stores, so L2 sees full-line writes.
// Requires whole stages (K % 128 == 0 for FP8 and FP6, K % 256 == 0 for FP4
// at SLAB = 128) and 4-byte aligned scale rows.  The library runs it for
// MXFP4 on 256 x 320 tiles only; every other whole-stage MX GEMM runs
// mxe_gemm_kernel.
template <int ELEM, int BM, int BN, int WM, int WN, int SLAB, int NS, int PK = 0>
__global__ __launch_bounds__(64 * WM * WN, 8 / (WM * WN) > 0 ? 8 / (WM * WN) : 1) void mxp_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ Ws, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int N,
    int K) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TJ = WTM / 32, TI = WTN / 32;  // 32 x 32 tiles per wave (M, N)
  constexpr int ROWS = BM + BN;
  constexpr int H = SLAB / 64;                 // 64-byte halves per slab
  constexpr int CPR = SLAB / 16;               // 16-byte chunks per row
  constexpr int RPG = 64 / CPR;                // rows per wave-wide code DMA
  constexpr int CODE_BYTES = ROWS * SLAB;
  constexpr bool FP4 = ELEM == 2;              // two codes per byte; else one code byte or FP6 slot byte per element
  constexpr int SDW = FP4 ? H : 1;             // scale dwords per row and stage
  constexpr int SGROUPS = ((ROWS * SDW + 63) / 64 + NW - 1) / NW * NW;  // wave-wide 4-byte scale DMAs per stage
  constexpr int STAGE = CODE_BYTES + SGROUPS * 256;
  constexpr int CGROUPS = CODE_BYTES / 1024;   // wave-wide 16-byte code DMAs per stage
  static_assert(SLAB == 64 || SLAB == 128, "slab");
  static_assert(NS >= 2 && NS <= 4, "stages");
  static_assert(CGROUPS % NW == 0 && SGROUPS % NW == 0, "DMA groups per wave");
  static_assert(BM % RPG == 0 && (BM * SDW) % 64 == 0, "a DMA group never straddles the A/W boundary");
  constexpr int CPW = CGROUPS / NW, SPW = SGROUPS / NW;
  constexpr int PER_WAVE = CPW + SPW;          // VMEM instructions per wave and stage
  constexpr int FMT = ELEM == 1 ? 0 : ELEM == 2 ? 4 : ELEM == 3 ? 2 : 3;  // E4M3, E2M1, E2M3, E3M2

  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[NS >= 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[NS == 4 ? STAGE : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 5, r32 = lane & 31;
  auto swz = [](int r) { return SLAB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  // Every operand row a lane reads is r32 plus a multiple of 32, which leaves
  // the swizzle unchanged: the lane's chunk offsets depend on (h, chunk) only
  // and the 32-row steps become immediate offsets of the LDS reads.
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BM % 32 == 0, "swizzle invariant under 32-row steps");
  const int sw0 = swz(r32);
  // FP8 / FP4: chunks 4h + q and 4h + 2 + q; FP6: the two chunks of 32-byte slot 2h + q (one K-block)
  auto choff = [&](int h, int c) { return ((ELEM >= 3 ? 4 * h + 2 * q + c : 4 * h + 2 * c + q) ^ sw0) << 4; };
  const int arow = (wm * WTM + r32) * SLAB, wrow = (BM + wn * WTN + r32) * SLAB;
  const int asrow = (wm * WTM + r32) * 4 * SDW, wsrow = (BM + wn * WTN + r32) * 4 * SDW;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  constexpr int GROUP = 8;
  const int group = (int)(id / (uint32_t)(GROUP * tiles_n));
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (int)(id % (uint32_t)gsz);
  const int tn = (int)((id % (uint32_t)(GROUP * tiles_n)) / (uint32_t)gsz);
  const int m0 = tm * BM, n0 = tn * BN;

  const int KB = FP4 ? K / 2 : K;
  const int SK = K / 32;
  const int nks = KB / SLAB;
  const uint32_t rows_a = (uint32_t)min(BM, M - m0), rows_w = (uint32_t)min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * KB, rows_a * (uint32_t)KB);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * KB, rows_w * (uint32_t)KB);
  // scale rows: row-major [rows, SK], or (PK) packed in 32-row groups, each
  // group's bytes stage-major: group g, stage s, row r: the SDW dwords at
  // g * 32 SK + s * 128 SDW + (r % 32) * 4 SDW, so that one stage's scales
  // of 32 rows are one contiguous run (m0 and n0 are multiples of 32)
  static_assert(BM % 32 == 0 && BN % 32 == 0, "whole 32-row scale groups per tile");
  const __amdgpu_buffer_rsrc_t rsa =
      PK ? make_rsrc(As + (size_t)m0 * SK, (rows_a + 31u) / 32u * 32u * (uint32_t)SK)
         : make_rsrc(As + (size_t)m0 * SK, rows_a * (uint32_t)SK);
  const __amdgpu_buffer_rsrc_t rsw =
      PK ? make_rsrc(Ws + (size_t)n0 * SK, (rows_w + 31u) / 32u * 32u * (uint32_t)SK)
         : make_rsrc(Ws + (size_t)n0 * SK, rows_w * (uint32_t)SK);

  // per-lane code DMA offsets without the K-step term: group g covers rows
  // RPG*g .. RPG*g+RPG-1, lane l row RPG*g + l/CPR, chunk l%CPR (swizzled)
  uint32_t coff[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int g = wave * CPW + u;
    const int r = g * RPG + lane / CPR;
    const int rr = (g * RPG < BM) ? r : r - BM;
    coff[u] = (uint32_t)rr * (uint32_t)KB + (uint32_t)(((lane % CPR) ^ swz(r)) << 4);
  }
  // per-lane scale DMA offsets without the K-step term: element e = row*SDW+d
  uint32_t soff[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int e = (wave * SPW + u) * 64 + lane;
    const int r = e / SDW, d = e % SDW;
    const int rr = r < BM ? r : r - BM;
    const uint32_t o = PK ? (uint32_t)(rr / 32) * 32u * (uint32_t)SK + (uint32_t)((rr % 32) * 4 * SDW + 4 * d)
                          : (uint32_t)rr * (uint32_t)SK + 4 * d;
    soff[u] = r < ROWS ? o : kOutOfRange;
  }
  // Stage arrays are passed by reference so that the DMA builtin sees the
  // __shared__ object itself (a runtime-selected or returned LDS pointer makes
  // the host pass drop the kernel's launch stub).
  auto issue = [&](auto& st, int ks) {
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int g = wave * CPW + u;
      lds_dma16(g * RPG < BM ? ra : rw, &st[g * 1024], coff[u], (uint32_t)(ks * SLAB));
    }
    // scale bytes of stage ks: FP8 / FP6 the dword of its 128 K-elements, FP4
    // the SDW dwords of its 64-byte halves; packed: the stage's run of 32 rows
    const uint32_t sk = PK ? (uint32_t)(ks * 128 * SDW)
                      : FP4 ? (uint32_t)(4 * SDW * ks) : (uint32_t)(4 * ((ks * SLAB) / 128));
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int gi = wave * SPW + u;
      // out-of-range rows carry offsets >= 2^31 and stay out of range
      lds_dma4((gi * 64) / SDW < BM ? rsa : rsw, &st[CODE_BYTES + gi * 256], soff[u], sk);
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  // A stage as one pipeline of H * TI MFMA groups (group g: W tile g % TI of
  // half g / TI against the TJ A tiles of that half): the LDS reads of group
  // g + 1 (with the A fragments of a half at its first group) are issued
  // ahead of the MFMAs of group g, and compiler fences keep that order, so
  // the reads of the next half overlap the last MFMAs of this one.  Scale
  // bytes are read per lane (byte loads): no VALU work sits between an LDS
  // read and its MFMA.
  auto stream_stage = [&](const auto& st, int ks) {
    constexpr int D = 1;
    constexpr int NSC = FP4 ? 2 : 1;
    constexpr int U = H * TI;
    const uint8_t* sb = st + CODE_BYTES;
    uint4 a[2][TJ][2], w[D + 1][2];
    uint32_t sa[2][TJ][NSC], sw[D + 1][NSC];
    auto read_group = [&](int g) {
      const int h = g / TI, i = g % TI;
      const int c = ks * H + h;
      const int b0 = FP4 ? 4 * h + q : 2 * (c & 1) + q;
      if (i == 0) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = wm * WTM + 32 * j + r32;
          const uint8_t* b = st + arow + 32 * j * SLAB;
          a[h & 1][j][0] = *reinterpret_cast<const uint4*>(b + choff(h, 0));
          a[h & 1][j][1] = *reinterpret_cast<const uint4*>(b + choff(h, 1));
#pragma unroll
          for (int e = 0; e < NSC; ++e) sa[h & 1][j][e] = sb[asrow + 32 * j * 4 * SDW + b0 + 2 * e];
        }
      }
      const int row = BM + wn * WTN + 32 * i + r32;
      const uint8_t* b = st + wrow + 32 * i * SLAB;
      const int sl = g % (D + 1);
      w[sl][0] = *reinterpret_cast<const uint4*>(b + choff(h, 0));
      w[sl][1] = *reinterpret_cast<const uint4*>(b + choff(h, 1));
#pragma unroll
      for (int e = 0; e < NSC; ++e) sw[sl][e] = sb[wsrow + 32 * i * 4 * SDW + b0 + 2 * e];
    };
    static_for<D>([&](auto gc) { read_group(decltype(gc)::value); });
    static_for<U>([&](auto uc) {
      constexpr int g = decltype(uc)::value;
      if constexpr (g + D < U) read_group(g + D);
      __builtin_amdgcn_sched_barrier(0);
      const int h = g / TI, i = g % TI, sl = g % (D + 1);
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (!FP4) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              as_v8i(w[sl][0], w[sl][1]), as_v8i(a[h & 1][j][0], a[h & 1][j][1]), acc[i][j], FMT, FMT, 0,
              (int)sw[sl][0], 0, (int)sa[h & 1][j][0]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              as_v8i_lo(w[sl][0]), as_v8i_lo(a[h & 1][j][0]), acc[i][j], FMT, FMT, 0, (int)sw[sl][0], 0,
              (int)sa[h & 1][j][0]);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              as_v8i_lo(w[sl][1]), as_v8i_lo(a[h & 1][j][1]), acc[i][j], FMT, FMT, 0, (int)sw[sl][1], 0,
              (int)sa[h & 1][j][1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // the wave's own DMA of a stage is complete when at most `pending` stages
  // issued after it are still in flight
  auto wait_own = [&](int pending) {
    if (pending >= 3) wait_vmcnt<3 * PER_WAVE < 64 ? 3 * PER_WAVE : 0>();
    else if (pending == 2) wait_vmcnt<2 * PER_WAVE < 64 ? 2 * PER_WAVE : 0>();
    else if (pending == 1) wait_vmcnt<PER_WAVE>();
    else wait_vmcnt<0>();
  };
  auto slot = [&](auto ic) -> decltype(auto) {
    constexpr int I = decltype(ic)::value;
    if constexpr (I == 0) return (st0);
    else if constexpr (I == 1) return (st1);
    else if constexpr (I == 2) return (st2);
    else return (st3);
  };

  // prologue: stages 0 .. NS-2 in flight
  static_for<NS - 1>([&](auto ic) {
    if (decltype(ic)::value < nks) issue(slot(ic), decltype(ic)::value);
  });
  // Step ks: own DMA of stage ks done -> barrier (every wave is past stage
  // ks-1) -> DMA stage ks+NS-1 into the slot of stage ks-1 -> MFMAs of stage
  // ks, one 64-byte half at a time.
  auto step = [&](auto u_c, int ks) {
    constexpr int u = decltype(u_c)::value;
    wait_own(min(NS - 2, nks - ks - 1));
    __builtin_amdgcn_s_barrier();
    if (ks + NS - 1 < nks) issue(slot(std::integral_constant<int, (u + NS - 1) % NS>{}), ks + NS - 1);
    stream_stage(slot(u_c), ks);
  };
  for (int ks = 0; ks < nks; ks += NS) {
    static_for<NS>([&](auto uc) {
      if (ks + decltype(uc)::value < nks) step(uc, ks + decltype(uc)::value);
    });
  }

  // ---- epilogue: (+ bias) -> bf16 RNE -> global
  constexpr int EPI_BYTES = 32 * (WTN * 2 + 16);
  constexpr int WPS = STAGE / EPI_BYTES;       // waves staged per stage array
  static_assert(WPS >= 1 && WPS * NS >= NW, "epilogue staging fits the stage buffers");
  // every wave is past its last LDS read and every DMA has landed
  __builtin_amdgcn_s_barrier();
  const int ea = wave / WPS;
  uint8_t* region = (ea == 0 ? st0 : ea == 1 ? st1 : ea == 2 ? st2 : st3) + (wave % WPS) * EPI_BYTES;
  store_tile_bf16<TI, TJ, WTM, WTN>(acc, 1.0f, region, bias, out, M, N, m0 + wm * WTM, n0 + wn * WTN, lane);
}

template <int ELEM, int BM, int BN, int WM, int WN, int SLAB, int NS, int PK = 0>
hipError_t launch_mxp(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as, const uint8_t* w,
                      const uint8_t* ws, const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((mxp_gemm_kernel<ELEM, BM, BN, WM, WN, SLAB, NS, PK>), dim3((unsigned)tiles),
                     dim3(64 * WM * WN), 0, stream, a, as, w, ws, bias, out, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// NVFP4 main path.  E2M1 codes with an E4M3 scale per 16 K-elements and a
// per-tensor fp32 scale on each operand.  The E4M3 block scale is not a power
// of two, so it cannot ride on the scaled MFMA's E8M0 port, and e2m1 * e4m3
// needs up to 6 significant bits, more than FP8 or FP4 hold; it lies in
// [2^-10, 2688] and is exact in f16.  So every code is dequantized in
// registers to f16 (v_cvt_scalef32_pk_f16_fp4 at unit scale, then one
// v_pk_mul_f16 by the block scale: measured on gfx950, the conversion's own
// fp32 scale operand applies only its power of two), fed to 32x32x16 f16
// MFMA with fp32 accumulators, and the tensor scales multiply the result.
//
// Tile, staging and epilogue follow the MX main path: 256 x 256 outputs, eight
// waves as 4 x 2, a two-stage LDS-DMA ring whose stage holds 128 code bytes
// (256 elements) per row plus that row's 16 scale bytes (one 16-byte DMA per
// row), loop-invariant per-lane DMA offsets with the K step in the scalar
// offset, and the LDS-staged bf16 epilogue.  Each operand dword (8 codes of
// one 16-element block) is dequantized once per stage and reused by every
// MFMA that needs it.  Lane (r, q) feeds the 16-K MFMA m (0..7) of the
// 64-byte half h with the 8 codes at elements 8 (m % 4) .. of 16-byte chunk
// 4h + q (m < 4) or 4h + 2 + q (m >= 4) of row r; A and W use the same K
// order, so the sum over K is unchanged.
// Requires K % 256 == 0 and 16-byte aligned scale rows.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 8 / (WM * WN) > 0 ? 8 / (WM * WN) : 1) void nv4_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ a_ts,
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, const float* __restrict__ w_ts,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int N, int K) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TJ = WTM / 32, TI = WTN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int SLAB = 128, H = 2;
  constexpr int CODE_BYTES = ROWS * SLAB;
  constexpr int STAGE = CODE_BYTES + ROWS * 16;
  constexpr int CGROUPS = CODE_BYTES / 1024, SGROUPS = ROWS * 16 / 1024;
  static_assert(CGROUPS % NW == 0 && SGROUPS % NW == 0 && BM % 64 == 0, "DMA groups");
  constexpr int CPW = CGROUPS / NW, SPW = SGROUPS / NW;

  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 5, r32 = lane & 31;
  auto swz = [](int r) { return (r >> 1) & 7; };

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  constexpr int GROUP = 8;
  const int group = (int)(id / (uint32_t)(GROUP * tiles_n));
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (int)(id % (uint32_t)gsz);
  const int tn = (int)((id % (uint32_t)(GROUP * tiles_n)) / (uint32_t)gsz);
  const int m0 = tm * BM, n0 = tn * BN;

  const int KB = K / 2, SK = K / 16;
  const int nks = KB / SLAB;
  const uint32_t rows_a = (uint32_t)min(BM, M - m0), rows_w = (uint32_t)min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * KB, rows_a * (uint32_t)KB);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * KB, rows_w * (uint32_t)KB);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(As + (size_t)m0 * SK, rows_a * (uint32_t)SK);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(Ws + (size_t)n0 * SK, rows_w * (uint32_t)SK);

  uint32_t coff[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int g = wave * CPW + u;
    const int r = g * 8 + lane / 8;
    const int rr = (g * 8 < BM) ? r : r - BM;
    coff[u] = (uint32_t)rr * (uint32_t)KB + (uint32_t)(((lane % 8) ^ swz(r)) << 4);
  }
  // scale DMA group gi: rows 64 gi .. 64 gi + 63, 16 bytes each
  uint32_t soff[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int r = (wave * SPW + u) * 64 + lane;
    soff[u] = (uint32_t)(r < BM ? r : r - BM) * (uint32_t)SK;
  }
  auto issue = [&](auto& st, int ks) {
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int g = wave * CPW + u;
      lds_dma16(g * 8 < BM ? ra : rw, &st[g * 1024], coff[u], (uint32_t)(ks * SLAB));
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int gi = wave * SPW + u;
      lds_dma16(gi * 64 < BM ? rsa : rsw, &st[CODE_BYTES + gi * 1024], soff[u], (uint32_t)(ks * 16));
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  // 8 codes (one dword) times a block scale -> one f16 MFMA operand
  auto deq = [](uint32_t x, h2 s) -> v8h {
    const h2 o0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s;
    const h2 o1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s;
    const h2 o2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s;
    const h2 o3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s;
    return v8h{o0.x, o0.y, o1.x, o1.y, o2.x, o2.y, o3.x, o3.y};
  };
  // one row's operands for a half: code chunks 4h+q, 4h+2+q and the E4M3
  // scales of their blocks (2q, 2q+1 of the half in sc[0], 4+2q, 5+2q in sc[1])
  struct RowOps {
    uint4 c[2];
    h2 sc[2];
  };
  auto read_row = [&](const auto& st, int row, int h, RowOps& o) {
    const uint8_t* b = st + row * SLAB;
    o.c[0] = *reinterpret_cast<const uint4*>(b + (((4 * h + q) ^ swz(row)) << 4));
    o.c[1] = *reinterpret_cast<const uint4*>(b + (((4 * h + 2 + q) ^ swz(row)) << 4));
    const uint2 s8 = *reinterpret_cast<const uint2*>(st + CODE_BYTES + row * 16 + 8 * h);
    o.sc[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8.x >> (16 * q), 1.0f, false);
    o.sc[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s8.y >> (16 * q), 1.0f, false);
  };
  auto operand = [&](const RowOps& o, int m) -> v8h {
    const uint4& c = o.c[m >> 2];
    const uint32_t x = ((m & 3) == 0) ? c.x : ((m & 3) == 1) ? c.y : ((m & 3) == 2) ? c.z : c.w;
    const _Float16 s = o.sc[m >> 2][(m & 3) >> 1];
    return deq(x, h2{s, s});
  };
  auto half_step = [&](const auto& st, int h) {
    RowOps ra_[TJ], rw_[TI];
#pragma unroll
    for (int j = 0; j < TJ; ++j) read_row(st, wm * WTM + 32 * j + r32, h, ra_[j]);
#pragma unroll
    for (int i = 0; i < TI; ++i) read_row(st, BM + wn * WTN + 32 * i + r32, h, rw_[i]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      v8h av[TJ], wv[TI];
#pragma unroll
      for (int j = 0; j < TJ; ++j) av[j] = operand(ra_[j], m);
#pragma unroll
      for (int i = 0; i < TI; ++i) wv[i] = operand(rw_[i], m);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[i], av[j], acc[i][j], 0, 0, 0);
    }
  };

  auto slot = [&](auto ic) -> decltype(auto) {
    if constexpr (decltype(ic)::value == 0) return (st0);
    else return (st1);
  };
  if (nks > 0) issue(st0, 0);
  // own DMA of stage ks done -> barrier (every wave is past stage ks-1) ->
  // DMA stage ks+1 into the other slot -> MFMAs of stage ks
  auto step = [&](auto u_c, int ks) {
    constexpr int u = decltype(u_c)::value;
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (ks + 1 < nks) issue(slot(std::integral_constant<int, 1 - u>{}), ks + 1);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      half_step(slot(u_c), h);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int ks = 0; ks < nks; ks += 2) {
    static_for<2>([&](auto uc) {
      if (ks + decltype(uc)::value < nks) step(uc, ks + decltype(uc)::value);
    });
  }

  // ---- epilogue: acc * ts_a * ts_w (+ bias) -> bf16 RNE -> global
  constexpr int EPI_BYTES = 32 * (WTN * 2 + 16);
  constexpr int WPS = STAGE / EPI_BYTES;
  static_assert(WPS >= 1 && WPS * 2 >= NW, "epilogue staging fits the stage buffers");
  __builtin_amdgcn_s_barrier();
  uint8_t* region = (wave / WPS == 0 ? st0 : st1) + (wave % WPS) * EPI_BYTES;
  store_tile_bf16<TI, TJ, WTM, WTN>(acc, a_ts[0] * w_ts[0], region, bias, out, M, N, m0 + wm * WTM, n0 + wn * WTN,
                                    lane);
}

// ---------------------------------------------------------------- skinny M
// out[m, n] for M <= MMAX activation rows: an HBM stream of W, bound by
// bandwidth (W is read once; 2 FLOP per 2 bytes per activation row).  The
// activations sit in LDS, padded with zero rows to MMAX, so the inner loop
// has no branch on M.  LPR lanes (8, 16 or 32) share one W row and read
// 16 * LPR contiguous bytes per instruction, so a wave-wide load covers whole
// lines; each lane keeps U such loads in flight, multiplies bf16 pairs with
// v_dot2_f32_bf16 (exact products, fp32 accumulation), and the partial sums
// of a row are combined with DPP lane permutes within each 16-lane row and
// a lane shuffle across rows.  64 / LPR W rows per wave: finer row groups
// spread N over the SIMDs more evenly.
template <int MMAX, int LPR>
__global__ __launch_bounds__(1024) void bf16_skinny_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ bias,
                                                          uint16_t* __restrict__ out, int M, int N, int K) {
  constexpr int U = 8;  // 16-byte W loads in flight per lane
  extern __shared__ uint4 sAv[];  // [MMAX][K/8], rows M .. MMAX - 1 zero
  const int kc = K / 8;
  for (int c = threadIdx.x; c < MMAX * kc; c += blockDim.x)
    sAv[c] = c < M * kc ? reinterpret_cast<const uint4*>(A)[c] : uint4{0u, 0u, 0u, 0u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  constexpr int RPW = 64 / LPR;                    // W rows per wave
  const int sub = lane % LPR;                      // lane within its row
  const int ngroups = (N + nwaves * RPW - 1) / (nwaves * RPW);
  // the workgroup's groups of nwaves * RPW W rows, grid-stride: the
  // activations are staged once per workgroup
  for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int n = (grp * nwaves + wave) * RPW + lane / LPR;
    const bool valid = n < N;
    const uint4* wrow = reinterpret_cast<const uint4*>(W + (size_t)(valid ? n : 0) * K);
    float acc[MMAX];
#pragma unroll
    for (int m = 0; m < MMAX; ++m) acc[m] = 0.f;
    auto dot8 = [](const uint4& w, const uint4& a, float c) {
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, a.x), c, false);
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, a.y), c, false);
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, a.z), c, false);
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, a.w), c, false);
      return c;
    };
    for (int c0 = sub; c0 < kc; c0 += LPR * U) {
      uint4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + LPR * u;
        x[u] = (valid && c < kc) ? wrow[c] : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + LPR * u;
        // a branch per W chunk (uniform except in the last chunk of K), which
        // also keeps the compiler from hoisting all U x MMAX activation reads
        if (c < kc) {
#pragma unroll
          for (int m = 0; m < MMAX; ++m) acc[m] = dot8(x[u], sAv[m * kc + c], acc[m]);
        }
      }
    }
    // sum over the 8 lanes of the row group: xor 1, xor 2 (quad permutes), then
    // the mirrored quad of the half row
    auto dpp_add = [](float v, int ctrl) {
      int o;
      if (ctrl == 0xB1) o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false);
      else if (ctrl == 0x4E) o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false);
      else o = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false);
      return v + __int_as_float(o);
    };
#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
      if (m < M) {
        float v = dpp_add(acc[m], 0xB1);
        v = dpp_add(v, 0x4E);
        v = dpp_add(v, 0x141);  // now the sum of each 8-lane half row
        if constexpr (LPR >= 16) v += __shfl_xor(v, 8, 64);
        if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
        if (sub == 0 && valid) {
          const float b = bias ? bf16_to_f32(bias[n]) : 0.f;
          out[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v + b);
        }
      }
    }
  }
}

// Skinny bf16 path: lanes per W row (each wave-wide load covers whole lines
// of 32 rows' 512-byte runs), the largest activation row count, and its
// activations' LDS bound (the whole LDS of a CU).
constexpr int kSkinnyLPR = 32;
constexpr int kSkinnyMaxRows = 16;
constexpr size_t kSkinnyMaxLds = 160 * 1024;

// Any K (row starts need not be 16-byte aligned): one thread per output.
__global__ __launch_bounds__(256) void bf16_generic_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ W,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ out, int M, int N, int K) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(bf16_to_f32(A[(size_t)m * K + k]), bf16_to_f32(W[(size_t)n * K + k]), s);
  if (bias) s += bf16_to_f32(bias[n]);
  out[idx] = (uint16_t)f32_to_bf16_rne(s);
}

}  // namespace

// Tile shapes of the generic path (BM activation rows x BN weight rows,
// WM x WN waves).
#ifndef MXQ_TILE_MX
#define MXQ_TILE_MX 256, 256, 2, 2
#endif
#ifndef MXQ_TILE_NV4
#define MXQ_TILE_NV4 128, 128, 2, 2
#endif
#ifndef MXQ_TILE_BF16
#define MXQ_TILE_BF16 256, 256, 2, 2
#endif


namespace {
// MXFP4 on 256 x 320 tiles, the one whole-stage MX GEMM the early-published
// kernel does not run (its registers do not fit them); PK: packed scale rows.
template <int PK>
hipError_t launch_mx4_wide(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as, const uint8_t* w,
                           const uint8_t* ws, const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  return launch_mxp<2, 256, 320, 4, 2, 128, 2, PK>(M, N, K, a, as, w, ws, bias, out, stream);
}
}  // namespace

hipError_t launch_mx_gemm(int elem, int packed, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                          const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  // whole 128-element FP8 / FP6 stages or 256-element FP4 stages and 4-byte
  // aligned scale rows: the 32x32x64 path with LDS-DMA staging
  const bool scales_aligned = (((uintptr_t)a_scales | (uintptr_t)w_scales) & 3) == 0;
  const bool whole_stages = K % (elem == 2 ? 256 : 128) == 0;
  // Tile width 256 or 320 columns (wave tiles 64 x 128 / 64 x 160): with one
  // workgroup per CU, the time is about (rounds of tiles) x (tile width), so
  // take the width with the smaller product; ties keep 256.
  // The early-published kernel (gemm_mx.hip) also takes 384 x 192 tiles
  // where their rounds fit the CUs better (mx_prefer_tall_tile).
  const int64_t cus = device_cu_count();
  const bool wide = mx_prefer_wide_tile(M, N, cus);
  const MxTile tile = mx_prefer_tall_tile(M, N, cus) ? MX_TILE_384x192 : wide ? MX_TILE_256x320 : MX_TILE_256x256;
  // the early-published kernel where it supports the tile, else (MXFP4 on
  // 256 x 320 tiles) mxp_gemm_kernel
  if (scales_aligned && whole_stages) {
    if (mx_staged_supports(elem, tile))
      return launch_mx_staged(elem, packed, tile, M, N, K, a_codes, a_scales, w_codes, w_scales, bias, out, stream);
    return packed ? launch_mx4_wide<1>(M, N, K, a_codes, a_scales, w_codes, w_scales, bias, out, stream)
                  : launch_mx4_wide<0>(M, N, K, a_codes, a_scales, w_codes, w_scales, bias, out, stream);
  }
  if (packed) return hipErrorInvalidValue;  // callers check the shape first
  if (elem >= 3) return hipErrorInvalidValue;  // FP6 has no generic path: callers check the shape first
  if (elem == 1)
    return launch_tiled<MX8, MXQ_TILE_MX>(M, N, K, a_codes, a_scales, w_codes, w_scales, nullptr, nullptr, bias,
                                             out, stream);
  return launch_tiled<MX4, MXQ_TILE_MX>(M, N, K, a_codes, a_scales, w_codes, w_scales, nullptr, nullptr, bias, out,
                                           stream);
}

bool mx_requant_supported(int elem, int64_t N, int64_t K, const uint8_t* a_scales, const uint8_t* w_scales) {
  const bool scales_aligned = (((uintptr_t)a_scales | (uintptr_t)w_scales) & 3) == 0;
  return scales_aligned && N % 32 == 0 && (elem == 2 ? K % 256 == 0 : K % 128 == 0);
}

hipError_t launch_mx_gemm_requant(int elem, int out_elem, int out_rceil, int act, int64_t M, int64_t N, int64_t K,
                                  const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                                  const uint8_t* w_scales, const uint16_t* bias, uint16_t* out_bf16,
                                  uint8_t* out_codes, uint8_t* out_scales, int64_t codes_ld, int64_t scales_ld,
                                  hipStream_t stream) {
  const int64_t qld = codes_ld ? codes_ld : (out_elem == 1 ? N : N / 2);
  const int64_t sld = scales_ld ? scales_ld : N / 32;
  // the tiles of the bf16-output GEMM; FP4 operands take 256 x 256 where it
  // would pick 256 x 320
  const int64_t cus = device_cu_count();
  MxTile tile = mx_prefer_tall_tile(M, N, cus)    ? MX_TILE_384x192
                : mx_prefer_wide_tile(M, N, cus) ? MX_TILE_256x320
                                                 : MX_TILE_256x256;
  if (!mx_staged_supports(elem, tile)) tile = MX_TILE_256x256;
  return launch_mx_staged_requant(elem, out_elem, out_rceil, act, tile, M, N, K, a_codes, a_scales, w_codes, w_scales,
                                  bias, out_bf16, out_codes, out_scales, qld, sld, stream);
}

hipError_t launch_nvfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_ts, const uint8_t* w_codes, const uint8_t* w_scales,
                             const float* w_ts, const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  // whole 256-element stages and 16-byte aligned scale rows: the 32x32x16 f16
  // path with LDS-DMA staging
  const bool scales_aligned = (((uintptr_t)a_scales | (uintptr_t)w_scales) & 15) == 0;
  if (K % 256 == 0 && scales_aligned) {
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    hipLaunchKernelGGL((nv4_gemm_kernel<256, 256, 4, 2>), dim3((unsigned)tiles), dim3(512), 0, stream, a_codes,
                       a_scales, a_ts, w_codes, w_scales, w_ts, bias, out, (int)M, (int)N, (int)K);
    return hipGetLastError();
  }
  return launch_tiled<NV4, MXQ_TILE_NV4>(M, N, K, a_codes, a_scales, w_codes, w_scales, a_ts, w_ts, bias, out,
                                           stream);
}

hipError_t launch_bf16_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* a, const uint16_t* w,
                            const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  if (K % 8 != 0) {
    const int64_t total = M * N;
    hipLaunchKernelGGL(bf16_generic_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a, w, bias,
                       out, (int)M, (int)N, (int)K);
    return hipGetLastError();
  }
  // up to 16 activation rows: the W stream of bf16_skinny_kernel with 4, 8
  // or 16 LDS activation rows (up to 160 KiB; above 64 KiB the kernel's
  // dynamic-LDS limit is raised first)
  const int mmax = M <= 4 ? 4 : M <= 8 ? 8 : 16;
  const size_t lds = (size_t)mmax * K * 2;
  if (M <= kSkinnyMaxRows && lds <= kSkinnyMaxLds) {
    // 4 waves per workgroup for up to 4 rows, 16 above (more waves share one
    // staged copy of the activations); as many workgroups as fit the CUs'
    // LDS, each looping over groups of W rows
    const int threads = mmax == 4 ? 256 : 1024;
    const int64_t rows_per_wg = (threads / 64) * (64 / kSkinnyLPR);
    const int64_t groups = (N + rows_per_wg - 1) / rows_per_wg;
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2048 / threads, (int64_t)(kSkinnyMaxLds / std::max<size_t>(lds, 1))));
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(groups, per_cu * device_cu_count()));
    auto run = [&](auto kern) -> hipError_t {
      if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, stream, a, w, bias, out, (int)M, (int)N, (int)K);
      return hipGetLastError();
    };
    if (mmax == 4) return run(&bf16_skinny_kernel<4, kSkinnyLPR>);
    if (mmax == 8) return run(&bf16_skinny_kernel<8, kSkinnyLPR>);
    return run(&bf16_skinny_kernel<16, kSkinnyLPR>);
  }
  return launch_tiled<BF16, MXQ_TILE_BF16>(M, N, K, a, nullptr, w, nullptr, nullptr, nullptr, bias, out, stream);
}

}  // namespace mxq
