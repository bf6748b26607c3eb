// MX block-scaled GEMM main path (MXFP8 / MXFP6 / MXFP4), the kernel every
// whole-stage MX GEMM of this library runs (bf16 output in gemm_mx.hip, the
// requantizing epilogue in gemm_mx_requant.hip): see mxe_gemm_kernel.
#pragma once

#include "gemm_tile.h"

namespace mxq {
namespace {

// ------------------------------------------------------------------------
// MX main path, early-published stages.  One BM x BN output tile per
// workgroup (256 x 256, 256 x 320 or 384 x 192), eight waves as 4 x 2 (e.g.
// 64 x 128 outputs each, 128 fp32 accumulators), scaled 32x32x64 MFMA, a
// two-stage LDS ring of 128-byte K slabs per row for both operands (128 FP8 /
// FP6-slot or 256 FP4 elements),
// filled by LDS DMA with the stage's scale dwords; 16-byte chunks
// XOR-swizzled by row (the LDS image of mxp_gemm_kernel).
//
// * Schedule.  A stage is U = 2 TI MFMA groups (half h, weight tile i: the
//   wave's TJ activation tiles of that half against weight tile i; U = 8 on
//   256 x 256 tiles).  The LDS reads of group g + D (D = 2 on 256 x 256, 1 on
//   the wider tiles) are issued before the MFMAs of group g.  The
//   barrier that publishes stage k+1 sits D groups before the end of stage k:
//   each wave first waits for its own DMA of stage k+1 and for its own reads
//   of stage k (all issued by then), so after the barrier the slot of stage k
//   takes the DMA of stage k+2, and the reads of stage k+1's first groups are
//   in flight while stage k's last 2D MFMAs run.
// * DMA spread.  A stage's DMA is issued a few instructions at a time between
//   MFMAs, not as one burst: a burst from every wave at once fills the
//   texture unit's command queue and stalls the issuing waves
//   (SQ_VMEM_TA_CMD_FIFO_FULL), and with them the matrix pipe.  The slot of
//   stage k is free from the barrier in stage k - 1 on, so stage k + 1's DMA
//   is split: its first SPL instructions go between the 2D MFMAs after that
//   barrier, the rest between the MFMAs of stage k's first E groups, which
//   leaves U - D - E groups for the last of them to land before the wait
//   that publishes the stage.  Measured on the FLUX MXFP8 shapes with
//   bit-identical outputs: 256 x 256 tiles 2-6 % faster with E = 2 than with
//   the whole DMA after the barrier (E = 3..6 lose it again), 256 x 320 tiles
//   5-8 % faster with E = 6 (E = 2: 2 %); MXFP4 2-3 % faster with E = 2;
//   384 x 192 tiles best with E = 3, with cold weights as with hot.
// * Scales.  One dword per row and stage holds the stage's four E8M0 bytes
//   (FP4: two dwords), one LDS read per tile and stage.  A lane shifts it
//   right by 8q and the MFMA's byte select picks the block: byte 2h is block
//   2h + q (FP8 / FP6), bytes 0 and 2 of dword h are blocks 4h + q and
//   4h + 2 + q (FP4).
// * Loop.  Stages run in pairs with no guard inside the loop body: a guarded
//   second stage makes the compiler carry the accumulators around it through
//   extra registers and scratch.  Every stage issues the same DMA, so the
//   waits count the same; near the end, and for the phantom stage of an odd
//   stage count, the DMA reads an empty buffer range: zero codes and zero
//   scales, whose MFMAs add exact zeros.
// * Measured on gfx950 against mxp_gemm_kernel at 256 x 256 tiles (same box,
//   alternating runs): 2-6 % faster on the FLUX shapes, bit-identical outputs.
//   Alternatives measured and dropped: activation fragments loaded straight
//   into registers (1.6x slower: in the MFMA operand layout one load covers
//   32 rows at 32 bytes each), and four waves of 128 x 128 with accumulators
//   in AGPRs (10-20 % slower although it needs a third less LDS traffic: with
//   one wave per SIMD every wait idles the matrix pipe).  Counters put the
//   FLUX MLP up-projection (384 x 192 tiles) at ~55 % MFMA busy at the
//   ~2.05 GHz the chip holds under this load.
// The accumulation order per output is that of mxp_gemm_kernel (stage by
// stage, half 0 then half 1), so both give identical outputs.  Requires
// whole stages (K % 128 == 0, FP4 K % 256 == 0) and 4-byte aligned scale
// rows.  REQ: 0 = bf16 output; 1 / 2 = the output MX-quantized to E4M3 /
// E2M1 codes and E8M0 scales (qcodes, qscales with row strides qld, sld;
// rceil selects the round-up shared-exponent rule), with the bf16 output also
// written when `out` is not null.  ACT: activation applied before the bf16
// rounding.  PK: both operands' scales in the packed layout.
template <int ELEM, int REQ = 0, int ACT = ACT_NONE, int PK = 0, int WM = 4, int WN = 2, int D = 2, int BN = 256, int E = 0, int BM = 256>
__global__ __launch_bounds__(64 * WM * WN, 1) void mxe_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ Ws, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int N,
    int K, uint8_t* __restrict__ qcodes, uint8_t* __restrict__ qscales, int rceil, int64_t qld, int64_t sld) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TJ = WTM / 32, TI = WTN / 32;  // activation / weight tiles of 32 rows per wave
  constexpr int ROWS = BM + BN;
  constexpr int SLAB = 128, H = 2, CPR = SLAB / 16, RPG = 64 / CPR;
  constexpr bool FP4 = ELEM == 2;
  constexpr int SDW = FP4 ? 2 : 1;              // scale dwords per row and stage
  constexpr int CODE_BYTES = ROWS * SLAB;
  constexpr int SGROUPS = ((ROWS * SDW + 63) / 64 + NW - 1) / NW * NW;
  constexpr int STAGE = CODE_BYTES + SGROUPS * 256;
  constexpr int CPW = CODE_BYTES / 1024 / NW, SPW = SGROUPS / NW;
  constexpr int U = H * TI;                     // MFMA groups per stage
  // weight register slots (groups in flight): the smallest divisor of U above
  // D, so that group g of every stage uses slot g % NSLOT
  constexpr int NSLOT = U % (D + 1) == 0 ? D + 1 : U % (D + 2) == 0 ? D + 2 : U % (D + 3) == 0 ? D + 3 : U;
  static_assert(U % NSLOT == 0 && D < NSLOT && D <= U / 2, "slot rotation");
  static_assert(BM % RPG == 0 && (BM * SDW) % 64 == 0, "a DMA group never straddles the A/W boundary");
  constexpr int FMT = ELEM == 1 ? 0 : ELEM == 2 ? 4 : ELEM == 3 ? 2 : 3;  // E4M3, E2M1, E2M3, E3M2

  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 5, r32 = lane & 31;
  auto swz = [](int r) { return (r >> 1) & 7; };
  const int sw0 = swz(r32);
  auto choff = [&](int h, int c) { return ((ELEM >= 3 ? 4 * h + 2 * q + c : 4 * h + 2 * c + q) ^ sw0) << 4; };
  const int arow = (wm * WTM + r32) * SLAB, wrow = (BM + wn * WTN + r32) * SLAB;
  const int asrow = CODE_BYTES + (wm * WTM + r32) * 4 * SDW, wsrow = CODE_BYTES + (BM + wn * WTN + r32) * 4 * SDW;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  // tiles grouped by GROUP M-tiles: 32 tiles in flight per XCD then span
  // 8 x 4 tiles (256-row tiles) or 4 x 8 (384 x 192: 3072 distinct rows per
  // round instead of 3840; measured 4 % faster with cold weights than 8)
  constexpr int GROUP = BM == 384 ? 4 : 8;
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
  // scale rows: row-major [rows, SK], or packed in 32-row groups with each
  // group's bytes stage-major (one stage of 32 rows = one 128 SDW-byte run)
  const __amdgpu_buffer_rsrc_t rsa =
      PK ? make_rsrc(As + (size_t)m0 * SK, (rows_a + 31u) / 32u * 32u * (uint32_t)SK)
         : make_rsrc(As + (size_t)m0 * SK, rows_a * (uint32_t)SK);
  const __amdgpu_buffer_rsrc_t rsw =
      PK ? make_rsrc(Ws + (size_t)n0 * SK, (rows_w + 31u) / 32u * 32u * (uint32_t)SK)
         : make_rsrc(Ws + (size_t)n0 * SK, rows_w * (uint32_t)SK);
  // a buffer range of no bytes: every load from it returns zeros
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(W, 0u);

  // per-lane code DMA offsets (stage 0): group g covers rows RPG g ..
  // RPG g + RPG - 1, lane l row RPG g + l / CPR, chunk l % CPR (swizzled)
  uint32_t coff[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int g = wave * CPW + u;
    const int r = g * RPG + lane / CPR;
    const int rr = (g * RPG < BM) ? r : r - BM;
    coff[u] = (uint32_t)rr * (uint32_t)KB + (uint32_t)(((lane % CPR) ^ swz(r)) << 4);
  }
  // per-lane scale DMA offsets (stage 0): element e = row * SDW + d
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
  // DMA of stage ks into `st`; valid == false: an empty range, zeros
  // DMA instructions t in [T0, T1) of stage ks into `st` (t < CPW: code
  // groups, then the scale groups); valid == false: an empty range, zeros
  auto issue_range = [&](auto& st, int ks, bool valid, auto t0_c, auto t1_c) {
    constexpr int T0 = decltype(t0_c)::value, T1 = decltype(t1_c)::value;
    const __amdgpu_buffer_rsrc_t ca = valid ? ra : rnone, cw = valid ? rw : rnone;
    const __amdgpu_buffer_rsrc_t sa = valid ? rsa : rnone, sw = valid ? rsw : rnone;
    const uint32_t kso = (uint32_t)(ks * SLAB);
    const uint32_t sk = PK ? (uint32_t)(ks * 128 * SDW) : (uint32_t)(4 * SDW * ks);
    static_for<T1 - T0>([&](auto tc) {
      constexpr int t = T0 + decltype(tc)::value;
      if constexpr (t < CPW) {
        const int g = wave * CPW + t;
        lds_dma16(g * RPG < BM ? ca : cw, &st[g * 1024], coff[t], kso);
      } else {
        const int gi = wave * SPW + (t - CPW);
        lds_dma4((gi * 64) / SDW < BM ? sa : sw, &st[CODE_BYTES + gi * 256], soff[t - CPW], sk);
      }
    });
  };
  constexpr int PER = CPW + SPW;  // DMA instructions per wave and stage
  // instructions [0, SPL) of a stage's DMA go after the barrier that frees
  // its slot, [SPL, PER) into the first E groups of the stage after it
  constexpr int SPL = E == 0 ? PER : (PER * D + D + E - 1) / (D + E);
  static_assert(E + D < U, "the stage's last DMA is issued before the wait that publishes it");
  auto issue = [&](auto& st, int ks, bool valid) {
    issue_range(st, ks, valid, std::integral_constant<int, 0>{}, std::integral_constant<int, PER>{});
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v16f{};

  uint4 a[H][TJ][2];         // activation chunks of each half
  uint32_t asc[2][TJ][SDW];  // activation scale dwords, by stage parity
  uint4 w[NSLOT][2];         // weight chunks, one slot per group in flight
  uint32_t wsc[2][TI][SDW];  // weight scale dwords, by stage parity and tile
  // LDS reads of group g of the stage in `st` (parity p): the weight chunks,
  // with the tile's first group its scale dword(s), and with a half's first
  // group the activation chunks of that half (and with the stage's first
  // group the activation scales)
  auto read_group = [&](const auto& st, auto p_c, auto g_c) {
    constexpr int p = decltype(p_c)::value, g = decltype(g_c)::value;
    constexpr int h = g / TI, i = g % TI, sl = g % NSLOT;
    if constexpr (i == 0) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint8_t* b = st + arow + 32 * j * SLAB;
        a[h][j][0] = *reinterpret_cast<const uint4*>(b + choff(h, 0));
        a[h][j][1] = *reinterpret_cast<const uint4*>(b + choff(h, 1));
        if constexpr (h == 0) {
          if constexpr (SDW == 1) {
            asc[p][j][0] = *reinterpret_cast<const uint32_t*>(st + asrow + 32 * j * 4 * SDW);
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(st + asrow + 32 * j * 4 * SDW);
            asc[p][j][0] = v.x;
            asc[p][j][1] = v.y;
          }
        }
      }
    }
    const uint8_t* b = st + wrow + 32 * i * SLAB;
    w[sl][0] = *reinterpret_cast<const uint4*>(b + choff(h, 0));
    w[sl][1] = *reinterpret_cast<const uint4*>(b + choff(h, 1));
    if constexpr (h == 0) {
      if constexpr (SDW == 1) {
        wsc[p][i][0] = *reinterpret_cast<const uint32_t*>(st + wsrow + 32 * i * 4 * SDW);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(st + wsrow + 32 * i * 4 * SDW);
        wsc[p][i][0] = v.x;
        wsc[p][i][1] = v.y;
      }
    }
  };
  auto mfma_group = [&](auto p_c, auto g_c, auto&& after) {
    constexpr int p = decltype(p_c)::value, g = decltype(g_c)::value;
    constexpr int h = g / TI, i = g % TI, sl = g % NSLOT;
    const int sh = 8 * q;
    static_for<TJ>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (!FP4) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            as_v8i(w[sl][0], w[sl][1]), as_v8i(a[h][j][0], a[h][j][1]), acc[i][j], FMT, FMT, 2 * h,
            (int)(wsc[p][i][0] >> sh), 2 * h, (int)(asc[p][j][0] >> sh));
      } else {
        const int sw = (int)(wsc[p][i][h] >> sh), sa = (int)(asc[p][j][h] >> sh);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8i_lo(w[sl][0]), as_v8i_lo(a[h][j][0]),
                                                                     acc[i][j], FMT, FMT, 0, sw, 0, sa);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8i_lo(w[sl][1]), as_v8i_lo(a[h][j][1]),
                                                                     acc[i][j], FMT, FMT, 2, sw, 2, sa);
      }
      after(jc);
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // prologue: stage 0 published, stage 1 in flight, stage 0's first reads.
  // The full wait also retires every scalar load of kernel arguments: one
  // still pending inside the loop (SMEM completes out of order) would turn
  // each LDS wait there into lgkmcnt(0).  The empty asm makes the epilogue's
  // arguments load here; left alone, the compiler issues their loads after
  // this wait and the first LDS wait of every loop pass becomes lgkmcnt(0).
  if constexpr (REQ == 0) {
    asm volatile("" ::"s"(bias), "s"(out));
  } else {
    asm volatile("" ::"s"(bias), "s"(out), "s"(qcodes), "s"(qscales), "s"(rceil), "s"(qld), "s"(sld));
  }
  issue(st0, 0, true);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  issue_range(st1, 1, nks > 1, std::integral_constant<int, 0>{}, std::integral_constant<int, SPL>{});
  static_for<D>([&](auto gc) { read_group(st0, I0{}, gc); });

  // Stage ks in slot p = ks % 2.
  auto step = [&](auto p_c, int ks_in) {
    constexpr int p = decltype(p_c)::value;
    using P1 = std::integral_constant<int, 1 - p>;
    auto& cur = [&]() -> auto& { if constexpr (p == 0) return st0; else return st1; }();
    auto& nxt = [&]() -> auto& { if constexpr (p == 0) return st1; else return st0; }();
    // the stage index is wave-uniform; without this the compiler may keep it
    // in a VGPR and wrap every DMA in a readfirstlane loop
    const int ks = __builtin_amdgcn_readfirstlane(ks_in);
    __builtin_amdgcn_sched_barrier(0);
    static_for<U>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + D < U) {
        read_group(cur, p_c, std::integral_constant<int, g + D>{});
      } else {
        if constexpr (g + D == U) {
          // own DMA of stage ks + 1 and own reads of stage ks complete, then
          // publish ks + 1; this slot then takes stage ks + 2
          wait_vmcnt<0>();
          wait_lgkmcnt0();
          __builtin_amdgcn_s_barrier();
        }
        read_group(nxt, P1{}, std::integral_constant<int, g + D - U>{});
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (g < E) {
        // the rest of stage ks + 1's DMA into the other slot, spread over
        // the MFMAs of this stage's first E groups
        constexpr int NH = E * TJ, s0 = g * TJ;
        mfma_group(p_c, gc, [&](auto jc) {
          constexpr int sl = s0 + decltype(jc)::value;
          issue_range(nxt, ks + 1, ks + 1 < nks, std::integral_constant<int, SPL + sl * (PER - SPL) / NH>{},
                      std::integral_constant<int, SPL + (sl + 1) * (PER - SPL) / NH>{});
        });
      } else if constexpr (g + D < U) {
        mfma_group(p_c, gc, [](auto) {});
      } else {
        // the first SPL DMA instructions of stage ks + 2 into this slot,
        // spread over the D * TJ MFMAs after the barrier
        constexpr int NSL = D * TJ, s0 = (g + D - U) * TJ;
        mfma_group(p_c, gc, [&](auto jc) {
          constexpr int sl = s0 + decltype(jc)::value;
          issue_range(cur, ks + 2, ks + 2 < nks, std::integral_constant<int, sl * SPL / NSL>{},
                      std::integral_constant<int, (sl + 1) * SPL / NSL>{});
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Stages in pairs with no guard inside the loop (a guarded second step
  // makes the compiler carry the accumulators through VGPRs around it).  With
  // an odd stage count the last pair's second stage reads only the empty
  // range: zero codes and scales, which add exact zeros.
  for (int ks = 0; ks < nks; ks += 2) {
    step(I0{}, ks);
    step(I1{}, ks + 1);
  }

  // ---- epilogue: (+ bias) -> bf16 RNE (or the requantized codes) -> global
  constexpr int EPI_BYTES = 32 * (WTN * 2 + 16);
  constexpr int WPS = STAGE / EPI_BYTES;  // waves staged per stage array
  static_assert(WPS * 2 >= NW, "epilogue staging fits the stage buffers");
  // every wave is past its last LDS read and every DMA has landed
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  uint8_t* region = (wave / WPS == 0 ? st0 : st1) + (wave % WPS) * EPI_BYTES;
  if constexpr (REQ == 0) {
    store_tile_bf16<TI, TJ, WTM, WTN, ACT>(acc, 1.0f, region, bias, out, M, N, m0 + wm * WTM, n0 + wn * WTN, lane);
  } else {
    store_tile_requant<TI, TJ, WTM, WTN, REQ, ACT>(acc, 1.0f, region, bias, qcodes, qscales, M, N, m0 + wm * WTM,
                                                   n0 + wn * WTN, lane, rceil, qld, sld);
    if (out) {
      wait_lgkmcnt0();
      __builtin_amdgcn_wave_barrier();
      store_tile_bf16<TI, TJ, WTM, WTN, ACT>(acc, 1.0f, region, bias, out, M, N, m0 + wm * WTM, n0 + wn * WTN,
                                             lane);
    }
  }
}

template <int ELEM, int REQ, int ACT, int PK, int BN, int D, int E, int BM = 256>
hipError_t launch_mxe(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as, const uint8_t* w,
                      const uint8_t* ws, const uint16_t* bias, uint16_t* out, hipStream_t stream, uint8_t* qcodes,
                      uint8_t* qscales, int rceil, int64_t qld, int64_t sld) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((mxe_gemm_kernel<ELEM, REQ, ACT, PK, 4, 2, D, BN, E, BM>), dim3((unsigned)tiles), dim3(512), 0, stream,
                     a, as, w, ws, bias, out, (int)M, (int)N, (int)K, qcodes, qscales, rceil, qld, sld);
  return hipGetLastError();
}

}  // namespace
}  // namespace mxq
