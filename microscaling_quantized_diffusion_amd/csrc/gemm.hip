// Tiled GEMMs on the gfx950 matrix cores, one kernel template for four
// operand modes:
//   MX8  : MXFP8 (E4M3 codes, E8M0 scale per 32 K)  -> scaled MFMA, FP8
//   MX4  : MXFP4 (E2M1 codes, E8M0 scale per 32 K)  -> scaled MFMA, FP4
//   NV4  : NVFP4 (E2M1 codes, E4M3 scale per 16 K, fp32 tensor scales)
//          -> codes dequantized in registers to f16 (exact) -> f16 MFMA
//   BF16 : unquantized bf16 operands                 -> bf16 MFMA
// computing out[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k] (+ bias[n]) with
// an fp32 accumulator and a nearest-even bf16 result.  This is the GEMM of
// the aitrends.kr MXFP8/NVFP4 article ("Section details": quantized weights
// times dynamically quantized activations; second "Evidence" block: small
// layers stay in bf16).
//
// Data flow per workgroup (one BM x BN output tile):
//   global --128-bit loads--> VGPR staging --ds_write_b128--> LDS (double
//   buffer; every row holds one 128-byte K slab; 16-byte chunks are XOR-
//   swizzled by row) --ds_read_b128--> MFMA operands.  Per-lane scales are
//   read from global memory one K step ahead.
//
// Operand layouts (measured on gfx950):
//   scaled 16x16x128: lane l serves row l % 16 and K-quarter q = l / 16;
//     FP8 operand bytes 0-15 = K [16q, 16q+16), bytes 16-31 = K [64+16q, +16);
//     FP4 operand bytes 0-15 = K [32q, 32q+32), low nibble first;
//     the scale byte of lane l is that of K-block q of row l % 16.
//   bf16/f16 16x16x32: lane l holds 8 K-values of row l % 16; any K order
//     works as long as both operands use the same one.
// Every mode therefore reads 16-byte chunks q and 4+q of each 128-byte row
// slab.  Weights are the MFMA "A" operand and activations the "B" operand,
// so the accumulators of lane l are 4 consecutive output columns of one
// output row (8-byte stores in the epilogue).
//
// NV4 dequantization: the E4M3 scale is not a power of two, so it cannot
// ride on the E8M0 scale port; e2m1 * e4m3 needs at most 6 significant
// bits and lies in [2^-10, 2688], so it is exact in f16.  Each dword of
// codes (8 elements, inside one 16-element block) is widened with
// v_cvt_scalef32_pk_f16_fp4 (unit scale) and multiplied by the block scale
// with v_pk_mul_f16; the tensor scales multiply the fp32 result.
#include "mxq_internal.h"

namespace mxq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

enum Mode { MX8 = 1, MX4 = 2, NV4 = 3, BF16 = 4 };

// XOR swizzle of the 16-byte chunk index by row: 16 rows reading the same
// logical chunk hit distinct banks with either 32 or 64 LDS banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ v8i as_v8i(const uint4& lo, const uint4& hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// FP4 operands use only the low four dwords.
__device__ __forceinline__ v8i as_v8i_lo(const uint4& lo) {
  const v4i v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

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

template <int MODE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ Ws, const float* __restrict__ a_ts, const float* __restrict__ w_ts,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int N, int K) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TJ = WTM / 16, TI = WTN / 16;  // 16x16 MFMA tiles per wave (M, N)
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile/threads mismatch");
  constexpr int LOADS_A = BM * 8 / NT, LOADS = (BM + BN) * 8 / NT;
  // scale bytes per lane per K step and row: MX8 1, MX4 2 (E8M0); NV4 4 (E4M3)
  constexpr int NSC = (MODE == MX8) ? 1 : (MODE == MX4) ? 2 : (MODE == NV4) ? 4 : 0;
  constexpr int NSC1 = NSC > 0 ? NSC : 1;
  constexpr int FMT = (MODE == MX8) ? 0 : 4;  // cbsz / blgp: 0 = FP8 E4M3, 4 = FP4 E2M1

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- global -> VGPR staging -> LDS
  uint4 stage[LOADS];
  auto load_step = [&](int ks) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const bool isA = u < LOADS_A;
      const int cc = isA ? tid + u * NT : tid + (u - LOADS_A) * NT;
      const int row = cc >> 3, ch = cc & 7;
      const int kb = ks * 128 + ch * 16;
      const int grow = (isA ? m0 : n0) + row;
      const bool ok = (grow < (isA ? M : N)) && (kb < KB);
      const uint8_t* src = (isA ? A : W) + (size_t)grow * KB + kb;
      stage[u] = ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_step = [&](int buf) {
    uint8_t* sA = smem + buf * (BM + BN) * 128;
    uint8_t* sW = sA + BM * 128;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const bool isA = u < LOADS_A;
      const int cc = isA ? tid + u * NT : tid + (u - LOADS_A) * NT;
      const int row = cc >> 3, ch = cc & 7;
      *reinterpret_cast<uint4*>((isA ? sA : sW) + row * 128 + ((ch ^ swz(row)) << 4)) = stage[u];
    }
  };

  // ---- per-lane scale bytes of one K step
  // MX: slot h -> K-block 4*MFMA_PER_STEP*ks + 4h + q.
  // NV4: slots {2q, 2q+1, 8+2q, 9+2q} of the step's 16 blocks (chunk q and 4+q).
  auto scale_block = [&](int ks, int h) -> int {
    if (MODE == NV4) return ks * 16 + (h >> 1) * 8 + 2 * q + (h & 1);
    return ks * (4 * NSC) + 4 * h + q;
  };
  int scW[TI][NSC1], scA[TJ][NSC1];
  auto load_scales = [&](int ks, int (&sw)[TI][NSC1], int (&sa)[TJ][NSC1]) {
    if (NSC == 0) return;
    const int pad = (MODE == NV4) ? 0 : 127;
#pragma unroll
    for (int h = 0; h < NSC; ++h) {
      const int kblk = scale_block(ks, h);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int n = n0 + wn * WTN + 16 * i + r16;
        sw[i][h] = (n < N && kblk < SK) ? (int)Ws[(size_t)n * SK + kblk] : pad;
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int m = m0 + wm * WTM + 16 * j + r16;
        sa[j][h] = (m < M && kblk < SK) ? (int)As[(size_t)m * SK + kblk] : pad;
      }
    }
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_step(0);
  load_scales(0, scW, scA);
  store_step(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const bool more = ks + 1 < nk;
    if (more) load_step(ks + 1);
    int nscW[TI][NSC1], nscA[TJ][NSC1];
    if (more) load_scales(ks + 1, nscW, nscA);

    const uint8_t* sA = smem + (ks & 1) * (BM + BN) * 128;
    const uint8_t* sW = sA + BM * 128;
    uint4 fw[TI][2], fa[TJ][2];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wn * WTN + 16 * i + r16;
      const uint8_t* base = sW + row * 128;
      fw[i][0] = *reinterpret_cast<const uint4*>(base + ((q ^ swz(row)) << 4));
      fw[i][1] = *reinterpret_cast<const uint4*>(base + (((4 + q) ^ swz(row)) << 4));
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int row = wm * WTM + 16 * j + r16;
      const uint8_t* base = sA + row * 128;
      fa[j][0] = *reinterpret_cast<const uint4*>(base + ((q ^ swz(row)) << 4));
      fa[j][1] = *reinterpret_cast<const uint4*>(base + (((4 + q) ^ swz(row)) << 4));
    }

    if constexpr (MODE == MX8) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              as_v8i(fw[i][0], fw[i][1]), as_v8i(fa[j][0], fa[j][1]), acc[i][j], FMT, FMT, 0, scW[i][0], 0,
              scA[j][0]);
    } else if constexpr (MODE == MX4) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                as_v8i_lo(fw[i][h]), as_v8i_lo(fa[j][h]), acc[i][j], FMT, FMT, 0, scW[i][h], 0, scA[j][h]);
    } else if constexpr (MODE == BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, fw[i][h]),
                                                                 __builtin_bit_cast(v8bf, fa[j][h]), acc[i][j], 0,
                                                                 0, 0);
    } else {  // NV4: 8 f16 MFMAs per step, one per dword d of (chunk q | chunk 4+q)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int half = d >> 2, dw = d & 3;
        const int slot = half * 2 + (dw >> 1);  // 16-element block of this dword
        v8h wa[TI], ab[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const uint32_t x = (dw == 0) ? fw[i][half].x : (dw == 1) ? fw[i][half].y : (dw == 2) ? fw[i][half].z
                                                                                             : fw[i][half].w;
          const _Float16 s = e4m3_to_f16((uint32_t)scW[i][slot]);
          h2 o[4];
          nv4_dequant_dword(x, h2{s, s}, o);
          wa[i] = v8h{o[0].x, o[0].y, o[1].x, o[1].y, o[2].x, o[2].y, o[3].x, o[3].y};
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const uint32_t x = (dw == 0) ? fa[j][half].x : (dw == 1) ? fa[j][half].y : (dw == 2) ? fa[j][half].z
                                                                                             : fa[j][half].w;
          const _Float16 s = e4m3_to_f16((uint32_t)scA[j][slot]);
          h2 o[4];
          nv4_dequant_dword(x, h2{s, s}, o);
          ab[j] = v8h{o[0].x, o[0].y, o[1].x, o[1].y, o[2].x, o[2].y, o[3].x, o[3].y};
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[i], ab[j], acc[i][j], 0, 0, 0);
      }
    }

    if (more) {
      store_step((ks + 1) & 1);
#pragma unroll
      for (int h = 0; h < NSC1; ++h) {
#pragma unroll
        for (int i = 0; i < TI; ++i) scW[i][h] = nscW[i][h];
#pragma unroll
        for (int j = 0; j < TJ; ++j) scA[j][h] = nscA[j][h];
      }
    }
    __syncthreads();
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
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<MODE, BM, BN, WM, WN>), dim3((unsigned)tiles), dim3(64 * WM * WN), 0, stream,
                     (const uint8_t*)a, as, (const uint8_t*)w, ws, a_ts, w_ts, bias, out, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

// ---------------------------------------------------------------- skinny M
// out[m, n] for M <= MMAX rows of activations: HBM-bound streaming of W.
// The activations sit in LDS; each wave walks whole W rows, lanes split K in
// 16-byte chunks, and a wave reduction produces M outputs per row.
template <int MMAX>
__global__ __launch_bounds__(256) void bf16_skinny_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ bias,
                                                          uint16_t* __restrict__ out, int M, int N, int K,
                                                          int rows_per_wg) {
  extern __shared__ uint4 sAv[];  // [M][K/8]
  const int kc = K / 8;
  for (int c = threadIdx.x; c < M * kc; c += 256) sAv[c] = reinterpret_cast<const uint4*>(A)[c];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_begin = blockIdx.x * rows_per_wg;
  const int n_end = min(N, n_begin + rows_per_wg);
  for (int n = n_begin + wave * 2; n < n_end; n += 8) {
    const bool two = n + 1 < n_end;
    float acc0[MMAX], acc1[MMAX];
#pragma unroll
    for (int m = 0; m < MMAX; ++m) acc0[m] = acc1[m] = 0.f;
    const uint4* w0 = reinterpret_cast<const uint4*>(W + (size_t)n * K);
    const uint4* w1 = reinterpret_cast<const uint4*>(W + (size_t)(two ? n + 1 : n) * K);
    for (int c = lane; c < kc; c += 64) {
      const uint4 x0 = w0[c], x1 = w1[c];
      const uint32_t wx0[4] = {x0.x, x0.y, x0.z, x0.w}, wx1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int m = 0; m < MMAX; ++m) {
        if (m < M) {
          const uint4 av = sAv[m * kc + c];
          const uint32_t ax[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float alo = __uint_as_float(ax[t] << 16), ahi = __uint_as_float(ax[t] & 0xFFFF0000u);
            acc0[m] = fmaf(alo, __uint_as_float(wx0[t] << 16), acc0[m]);
            acc0[m] = fmaf(ahi, __uint_as_float(wx0[t] & 0xFFFF0000u), acc0[m]);
            acc1[m] = fmaf(alo, __uint_as_float(wx1[t] << 16), acc1[m]);
            acc1[m] = fmaf(ahi, __uint_as_float(wx1[t] & 0xFFFF0000u), acc1[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
      if (m < M) {
        float s0 = acc0[m], s1 = acc1[m];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          s0 += __shfl_xor(s0, off, 64);
          s1 += __shfl_xor(s1, off, 64);
        }
        if (lane == 0) {
          const float b0 = bias ? bf16_to_f32(bias[n]) : 0.f;
          out[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(s0 + b0);
          if (two) {
            const float b1 = bias ? bf16_to_f32(bias[n + 1]) : 0.f;
            out[(size_t)m * N + n + 1] = (uint16_t)f32_to_bf16_rne(s1 + b1);
          }
        }
      }
    }
  }
}

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

hipError_t launch_mx_gemm(int elem, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                          const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  if (elem == 1)
    return launch_tiled<MX8, 128, 128, 2, 2>(M, N, K, a_codes, a_scales, w_codes, w_scales, nullptr, nullptr, bias,
                                             out, stream);
  return launch_tiled<MX4, 128, 128, 2, 2>(M, N, K, a_codes, a_scales, w_codes, w_scales, nullptr, nullptr, bias, out,
                                           stream);
}

hipError_t launch_nvfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_ts, const uint8_t* w_codes, const uint8_t* w_scales,
                             const float* w_ts, const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  return launch_tiled<NV4, 128, 128, 2, 2>(M, N, K, a_codes, a_scales, w_codes, w_scales, a_ts, w_ts, bias, out,
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
  const size_t lds = (size_t)M * K * 2;
  if (M <= 16 && lds <= 64 * 1024) {
    const int rows_per_wg = 32;
    const unsigned grid = (unsigned)((N + rows_per_wg - 1) / rows_per_wg);
    if (M <= 4)
      hipLaunchKernelGGL(bf16_skinny_kernel<4>, dim3(grid), dim3(256), lds, stream, a, w, bias, out, (int)M, (int)N,
                         (int)K, rows_per_wg);
    else
      hipLaunchKernelGGL(bf16_skinny_kernel<16>, dim3(grid), dim3(256), lds, stream, a, w, bias, out, (int)M, (int)N,
                         (int)K, rows_per_wg);
    return hipGetLastError();
  }
  return launch_tiled<BF16, 128, 128, 2, 2>(M, N, K, a, nullptr, w, nullptr, nullptr, nullptr, bias, out, stream);
}

}  // namespace mxq
