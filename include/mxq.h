/*
 * mxq.h -- C ABI of the microscaling-quantized GEMM library for MI355X (gfx950).
 *
 * The library quantizes bf16 activations into block-scaled ("microscaling")
 * formats and multiplies them with pre-quantized weights on the GPU, the
 * inference recipe of the aitrends.kr article "Accelerating diffusion-model
 * inference with MXFP8 and NVFP4 quantization on NVIDIA B200":
 *   - "Section details": weights quantized once when the pipeline is loaded,
 *     activations quantized dynamically on every call (the TorchAO
 *     NVFP4 dynamic-activation / NVFP4-weight configuration);
 *   - Glossary "Microscaling Formats": a block of 16-32 elements shares one
 *     scale; "MXFP8": the OCP standard 8-bit format; "NVFP4": 4-bit format;
 *   - second "Evidence" block: layers with min(M, K, N) < 1024 stay in bf16.
 * Element / scale encodings follow the OCP Microscaling Formats v1.0
 * specification, which the Glossary entry for MXFP8 names.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - GEMM: out[M, N] = A[M, K] * W[N, K]^T (+ bias[N]); W is a linear layer's
 *    weight stored out-features by in-features.  Blocks run along K.
 *  - Layouts are dense row-major with K innermost:
 *      bf16 A [M, K], W [N, K], out [M, N], bias [N];
 *      MXFP8 codes  uint8 [rows, K]     E4M3, scales uint8 [rows, K/32] E8M0;
 *      MXFP4 codes  uint8 [rows, K/2]   E2M1, element 2j in the low nibble of
 *                                        byte j; scales uint8 [rows, K/32] E8M0;
 *      NVFP4 codes  uint8 [rows, K/2]   E2M1 (same packing), scales uint8
 *                                        [rows, K/16] E4M3, plus one float32
 *                                        per-tensor scale in device memory;
 *      MXFP6 codes  uint8 [rows, K]     E2M3 or E3M2: each 32-element block
 *                                        takes a 32-byte slot, the 24 bytes of
 *                                        its little-endian 192-bit integer
 *                                        (element j at bits 6j..6j+5), then 8
 *                                        zero bytes; scales uint8 [rows, K/32]
 *                                        E8M0.  The MXFP6 GEMM needs K % 128
 *                                        == 0 (MXQ_ERR_UNSUPPORTED otherwise)
 *                                        and 4-byte aligned scale pointers
 *                                        (MXQ_ERR_ALIGN); MXFP6 codes are
 *                                        GEMM operands, not a requantized
 *                                        output format.
 *  - Every pointer is caller-owned DEVICE memory (the library never
 *    allocates or frees).  Base pointers of A, W, codes, out and workspace
 *    must be 16-byte aligned; scale and bias pointers need no alignment
 *    (except the MXFP6 GEMM's scales, above).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    stream-ordered and return before the GPU work completes; device faults
 *    surface at the caller's next synchronisation.  Calls on different
 *    streams with disjoint outputs and workspaces may run concurrently.
 *  - Arguments are validated on the host before anything is enqueued, in
 *    the order format, sizes, pointers, alignment, workspace; on any error
 *    nothing is launched.  M == 0 or N == 0 (or rows == 0) is a successful
 *    no-op, decided right after the sizes, so empty tensors may pass NULL
 *    pointers (an NVFP4 quantization of zero rows writes no tensor scale).
 *    K must be a positive multiple of the block size (32 for MX formats, 16
 *    for NVFP4) wherever K is used.
 *  - No state between calls beyond a per-device cache of the compute-unit
 *    count (used to pick the GEMM tile width).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 9

typedef enum {
  MXQ_FMT_MXFP8 = 1, /* E4M3 codes, E8M0 scale per 32 K-elements */
  MXQ_FMT_MXFP4 = 2, /* E2M1 codes, E8M0 scale per 32 K-elements */
  MXQ_FMT_NVFP4 = 3, /* E2M1 codes, E4M3 scale per 16 K-elements, fp32 per-tensor scale */
  MXQ_FMT_MXFP6_E2M3 = 4, /* E2M3 codes, E8M0 scale per 32 K-elements */
  MXQ_FMT_MXFP6_E3M2 = 5  /* E3M2 codes, E8M0 scale per 32 K-elements */
} mxq_format;

/*
 * Shared-scale rule flag, OR-ed into the format argument of a call that
 * quantizes to an MX format: mxq_quantize, mxq_quant_gemm_fused, and the
 * out_fmt of mxq_gemm_requant.
 *   without it        e = floor(log2 amax) - emax (the OCP MX v1.0 rule the
 *                     aitrends.kr article's Glossary entry "MXFP8" names); a
 *                     block maximum above the element range saturates;
 *   MXQ_SCALE_RCEIL   e = ceil(log2(amax / max_elem)), max_elem = 448 (E4M3)
 *                     or 6 (E2M1): the smallest power of two that keeps the
 *                     block maximum in range, so no element saturates.
 * Either way e is clamped to [-127, 127].  The rule does not change the code
 * or scale formats: mxq_gemm and the input format of mxq_gemm_requant accept
 * and ignore the flag, and mxq_workspace_bytes ignores it.  With
 * MXQ_FMT_NVFP4, or with a bit other than the two flags here, a call returns
 * MXQ_ERR_FORMAT.
 */
#define MXQ_SCALE_RCEIL 0x100

/*
 * Packed scale layout flag (MX formats; a storage layout of our own, the
 * weight pre-packing of a deployment: the pages fix no scale layout).  An MX
 * scale tensor of `rows` rows and S = K/32 blocks per row is normally
 * row-major [rows, S].  Packed, rows are padded to R = 32 * ceil(rows / 32)
 * (R * S bytes, padding bytes unspecified) and block kb of row r sits at
 *   (r / 32) * 32 S + (kb / P) * 32 P + (r % 32) * P + kb % P,
 * P = 4 (MXFP8, MXFP6) or 8 (MXFP4): for each group of 32 rows, the scales
 * of one GEMM K stage (128 / 256 elements) are one contiguous run, which the
 * GEMM fetches in whole cache lines.  Needs K a multiple of 32 P and
 * R * S < 2^32 (MXQ_ERR_UNSUPPORTED otherwise).  Meaning per call:
 *   mxq_quantize           writes the scales packed;
 *   mxq_gemm               both operands' scales are packed (4-byte aligned);
 *   mxq_quant_gemm_fused   W's scales are packed (4-byte aligned); A is
 *                          quantized into the workspace packed as well;
 *   mxq_workspace_bytes    ignored;
 * every other call returns MXQ_ERR_FORMAT for it, as does MXQ_FMT_NVFP4.
 * Codes are unchanged, and results equal those of the row-major layout bit
 * for bit.
 */
#define MXQ_SCALES_PACKED 0x200

typedef enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = 1,        /* a required pointer is NULL */
  MXQ_ERR_FORMAT = 2,      /* unknown mxq_format */
  MXQ_ERR_SHAPE = 3,       /* negative size, K not a positive multiple of the block, or a
                              GEMM beyond K <= 2^22 / M * N <= 2^39 */
  MXQ_ERR_ALIGN = 4,       /* a 16-byte-aligned pointer is misaligned */
  MXQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than mxq_workspace_bytes() */
  MXQ_ERR_UNSUPPORTED = 6, /* valid request this build does not implement */
  MXQ_ERR_LAUNCH = 7,      /* a kernel launch failed (hipGetLastError after launch) */
  MXQ_ERR_TOO_LARGE = 8    /* the problem needs more than the library's fixed scratch array
                              (mxq_quant_gemm_fused_noalloc) */
} mxq_status;

/*
 * Quantize a bf16 matrix x [rows, cols] along cols (dynamic activation
 * quantization, and the offline weight quantization of the same article's
 * "Section details").
 *
 * MX formats (OCP MX v1.0 shared exponent): per block of 32, amax = max|x|,
 * e = clamp(floor(log2 amax) - emax, -127, 127) with emax = 8 (E4M3), 2 (E2M1,
 * E2M3) or 4 (E3M2), e = -127 for an all-zero block; scale byte = e + 127;
 * codes are x / 2^e rounded to nearest-even with saturation at +-448 / +-6 /
 * +-7.5 / +-28 (never NaN); signed zeros keep their sign.  A block holding NaN/Inf gets scale 0xFF and
 * zero codes.  With MXQ_SCALE_RCEIL, e = clamp(ceil(log2(amax / max_elem)),
 * -127, 127) instead.
 *
 * NVFP4: ts = RN_fp32(G / 2688) with G = max|x| over the whole tensor
 * (G = 0 gives ts = 1); per block of 16 with amax B, the E4M3 scale is the
 * round-to-nearest-even (saturating) encoding of B / (6 ts), raised to 0x01
 * if it rounds to zero, and 0x00 for an all-zero block; codes are the E2M1
 * encoding of x / (dec(scale) * ts), each quotient rounded once.  Any NaN/Inf
 * in the tensor gives ts = NaN, scales 0x7F and zero codes.
 *
 *   fmt            MXQ_FMT_*, MX formats optionally | MXQ_SCALE_RCEIL and / or
 *                  | MXQ_SCALES_PACKED
 *   x_bf16         device, bf16 [rows, cols], 16-byte aligned
 *   rows, cols     rows >= 0; cols a positive multiple of the block size
 *   codes          device, out: uint8 [rows, cols] (MXFP8, MXFP6) or
 *                  [rows, cols/2] (FP4)
 *   scales         device, out: uint8 [rows, cols/32] (MX; packed:
 *                  [32 ceil(rows/32), cols/32]) or [rows, cols/16] (NVFP4)
 *   tensor_scale   device float[1], out (NVFP4, required); must be NULL for MX
 *   workspace      device scratch of mxq_workspace_bytes(fmt, rows, cols, 0)
 *                  bytes (0 for MX, where it may be NULL)
 *   stream         hipStream_t
 */
mxq_status mxq_quantize(mxq_format fmt, const void* x_bf16, int64_t rows, int64_t cols, void* codes,
                        void* scales, float* tensor_scale, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Block-scaled GEMM on already-quantized operands:
 *   out[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k] (+ bias[n]), rounded to bf16
 * (nearest-even) from an fp32 accumulator.  deq is the format's decoding
 * (MX: code * 2^(scale-127); NVFP4: code * dec_E4M3(scale) * tensor scale).
 * This is the low-precision GEMM of the article's "Section details".
 *
 *   a_codes/a_scales   device, A quantized as by mxq_quantize (rows = M)
 *   a_tensor_scale     device float[1] (NVFP4, required); NULL for MX
 *   w_codes/w_scales   device, W [N, K] quantized (rows = N)
 *   w_tensor_scale     device float[1] (NVFP4, required); NULL for MX
 *   bias_bf16          device bf16 [N] or NULL
 *   out_bf16           device bf16 [M, N], 16-byte aligned
 * Sizes: M, N >= 0 with M * N <= 2^39, K a positive multiple of the block and
 * at most 2^22 (a tile's rows of codes stay within one 32-bit buffer range);
 * anything else returns MXQ_ERR_SHAPE before any launch.
 */
mxq_status mxq_gemm(mxq_format fmt, int64_t M, int64_t N, int64_t K, const void* a_codes, const void* a_scales,
                    const float* a_tensor_scale, const void* w_codes, const void* w_scales,
                    const float* w_tensor_scale, const void* bias_bf16, void* out_bf16, void* stream);

/*
 * Dynamic activation quantization followed by the block-scaled GEMM, in one
 * call: A (bf16) is quantized once into `workspace`, then multiplied with the
 * pre-quantized W.  Results are identical to mxq_quantize + mxq_gemm with the
 * same fmt (an MXQ_SCALE_RCEIL flag selects A's scale rule).
 *
 *   a_bf16         device bf16 [M, K], 16-byte aligned
 *   w_*            as in mxq_gemm
 *   workspace      device scratch, at least mxq_workspace_bytes(fmt, M, K, 1)
 *                  bytes, 16-byte aligned; its contents are overwritten
 * Sizes as in mxq_gemm.
 */
mxq_status mxq_quant_gemm_fused(mxq_format fmt, int64_t M, int64_t N, int64_t K, const void* a_bf16,
                                const void* w_codes, const void* w_scales, const float* w_tensor_scale,
                                const void* bias_bf16, void* out_bf16, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * mxq_quant_gemm_fused without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The activation codes and scales go into
 * a fixed array inside the library, MXQ_NOALLOC_SCRATCH_BYTES on each GPU the
 * library runs on, held until the process ends; the call allocates and frees
 * nothing (the first call on a device only looks up the array's device
 * address).  Arguments, checks and results are those of
 * mxq_quant_gemm_fused with the same arguments, bit for bit; a problem whose
 * mxq_workspace_bytes(fmt, M, K, 1) exceeds MXQ_NOALLOC_SCRATCH_BYTES returns
 * MXQ_ERR_TOO_LARGE before any launch.  Every call on one GPU uses that GPU's
 * one array and leaves its contents behind: calls that overlap on the same
 * GPU (other streams, other host threads) race, and the caller must order
 * them.
 */
#define MXQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mxq_status mxq_quant_gemm_fused_noalloc(mxq_format fmt, int64_t M, int64_t N, int64_t K, const void* a_bf16,
                                        const void* w_codes, const void* w_scales, const float* w_tensor_scale,
                                        const void* bias_bf16, void* out_bf16, void* stream);

/*
 * Block-scaled GEMM whose epilogue emits the next layer's MX-quantized
 * activations (producer-fused quantization; the devin.kr article on FLUX
 * image generation accelerated 4.45x on Blackwell, "Compute efficiency and
 * acceleration": fused activation kernels around the low-precision GEMMs):
 *   y = act(deq(A) deq(W)^T + bias) formed in fp32 and rounded to bf16
 *   (nearest even), then quantized along N in 32-column blocks exactly as
 *   mxq_quantize(out_fmt, y) would, so the codes feed the next mxq_gemm as
 *   its A operand without y passing through memory as bf16.
 *   act: 0 = none, 1 = GELU in its tanh form,
 *        0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))).
 *
 *   fmt, M, N, K, a_*, w_*, bias_bf16   as in mxq_gemm (MXFP8, MXFP6 or MXFP4)
 *   out_fmt        MXQ_FMT_MXFP8 or MXQ_FMT_MXFP4, optionally | MXQ_SCALE_RCEIL
 *   out_bf16       device bf16 [M, N], 16-byte aligned, or NULL: also store y
 *   out_codes      device, out: uint8 [M, N] (MXFP8) or [M, N/2] (MXFP4),
 *                  rows out_codes_ld bytes apart, 16-byte aligned
 *   out_scales     device, out: uint8 [M, N/32] E8M0, rows out_scales_ld
 *                  bytes apart
 *   out_codes_ld, out_scales_ld   row strides in bytes, 0 for dense rows;
 *                  otherwise at least a dense row, the codes' a multiple of
 *                  16 (MXQ_ERR_SHAPE / MXQ_ERR_ALIGN).  With them the GEMM
 *                  writes a column range of a wider quantized matrix (pass
 *                  pointers offset to its first column, a multiple of 32
 *                  elements), e.g. one part of a concatenated activation.
 * Supported where N % 32 == 0, K % 128 == 0 (MXFP8 and MXFP6 operands) or
 * K % 256 == 0 (MXFP4 operands), and the scale rows are 4-byte aligned; other
 * shapes, and MXFP6 or NVFP4 as out_fmt, return MXQ_ERR_UNSUPPORTED.  Sizes
 * otherwise as in mxq_gemm.
 */
mxq_status mxq_gemm_requant(mxq_format fmt, int64_t M, int64_t N, int64_t K, const void* a_codes,
                            const void* a_scales, const void* w_codes, const void* w_scales, const void* bias_bf16,
                            int act, mxq_format out_fmt, void* out_bf16, void* out_codes, void* out_scales,
                            int64_t out_codes_ld, int64_t out_scales_ld, void* stream);

/*
 * bf16 GEMM for layers left unquantized by the selective rule:
 *   out[m, n] = sum_k A[m, k] * W[n, k] (+ bias[n]) with bf16 inputs, an fp32
 * accumulator and a nearest-even bf16 result.  1 <= K <= 2^22 (no block
 * constraint), M * N <= 2^39.
 *   a_bf16 [M, K], w_bf16 [N, K], out_bf16 [M, N]: device, 16-byte aligned.
 */
mxq_status mxq_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* a_bf16, const void* w_bf16,
                         const void* bias_bf16, void* out_bf16, void* stream);

/*
 * Block-scaled FP8 attention, for each of the B * H heads independently:
 *   out = softmax(Q K^T / sqrt(D)) V computed in 8-bit floating point, the
 * FP8 attention with per-token error correction of the devin.kr article on
 * FLUX image generation accelerated on Blackwell ("Compute efficiency and
 * acceleration"), read as follows (the pages give no steps):
 *   - Q and K are MXFP8-quantized along D (E4M3 codes, one E8M0 scale per 32
 *     channels of each token, the rule of mxq_quantize); V is
 *     MXFP8-quantized along the token axis (one scale per 32 tokens of each
 *     channel);
 *   - scores come from the dequantized codes with an fp32 accumulator; the
 *     softmax runs online over key tiles of 64 in key order: running max m,
 *     p = exp(s - m) <= 1 encoded as E4M3 at the fixed scale 2^8, the output
 *     accumulator and the row sum (of the unquantized p) rescaled by
 *     exp(m_old - m_new) at each tile; out = acc / sum, rounded to bf16
 *     (nearest-even).
 * All the quantization happens inside the call, into `workspace`.
 *
 *   B, H, S, D     batch, heads, tokens (queries = keys), head dimension
 *   q_bf16, k_bf16, v_bf16   device bf16 [B, H, S, D], 16-byte aligned
 *   out_bf16       device bf16 [B, H, S, D], 16-byte aligned
 *   workspace      device scratch of mxq_attention_workspace_bytes(B, H, S, D)
 *                  bytes, 16-byte aligned; its contents are overwritten
 * Sizes: B, H, S >= 0, D > 0, S <= 2^24, B * H <= 65535, else MXQ_ERR_SHAPE.
 * This build implements D == 128 with S a multiple of 64; other valid sizes
 * return MXQ_ERR_UNSUPPORTED.  B * H == 0 or S == 0 is a successful no-op.
 * Inputs are expected finite (a NaN or Inf makes its head's output
 * meaningless).
 */
mxq_status mxq_attention_fp8(int64_t B, int64_t H, int64_t S, int64_t D, const void* q_bf16, const void* k_bf16,
                             const void* v_bf16, void* out_bf16, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * mxq_attention_fp8 with the output MX-quantized for the next layer instead
 * of stored as bf16, so that no bf16 attention output passes through memory
 * on its way to a quantized linear: the bf16 values mxq_attention_fp8 would
 * store are quantized as mxq_quantize(out_fmt) would quantize them, laid out
 * token-major with the heads side by side, the layout a DiT's output
 * projection reads:
 *   row b * S + s, column h * D + d  (B * S rows, H * D columns).
 *
 *   B, H, S, D, q_bf16, k_bf16, v_bf16, workspace   as in mxq_attention_fp8
 *   out_fmt        MXQ_FMT_MXFP8 or MXQ_FMT_MXFP4, optionally | MXQ_SCALE_RCEIL
 *   out_codes      device, out: uint8 rows of H * D (MXFP8) or H * D / 2 (MXFP4)
 *                  bytes, out_codes_ld bytes apart, 16-byte aligned
 *   out_scales     device, out: uint8 rows of H * D / 32 E8M0 bytes,
 *                  out_scales_ld bytes apart
 *   out_codes_ld, out_scales_ld   row strides in bytes, 0 for dense rows, as
 *                  in mxq_gemm_requant (so the codes can land in a column
 *                  range of a wider matrix, e.g. a concatenated activation)
 * Errors as in mxq_attention_fp8; NVFP4 output is MXQ_ERR_UNSUPPORTED.
 */
mxq_status mxq_attention_fp8_requant(int64_t B, int64_t H, int64_t S, int64_t D, const void* q_bf16,
                                     const void* k_bf16, const void* v_bf16, mxq_format out_fmt,
                                     void* out_codes, void* out_scales, int64_t out_codes_ld,
                                     int64_t out_scales_ld, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes needed by mxq_attention_fp8; 0 for sizes it rejects. */
size_t mxq_attention_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D);

/*
 * Workspace bytes needed by mxq_quantize (fused = 0) or mxq_quant_gemm_fused
 * (fused = 1) for an [M, K] activation.  Returns 0 for invalid arguments and
 * for MX quantization (which needs none).
 */
size_t mxq_workspace_bytes(mxq_format fmt, int64_t M, int64_t K, int fused);

/*
 * Selective quantization rule: 1 iff min(M, K, N) >= 1024, else 0 (layers
 * too small for quantization to pay off stay bf16; aitrends.kr article,
 * second "Evidence" block).  Advisory: callers choose the entry point.
 */
int mxq_should_quantize(int64_t M, int64_t K, int64_t N);

/* Static description of a status code; never NULL. */
const char* mxq_status_string(mxq_status s);

/* MXQ_ABI_VERSION of the loaded library. */
int mxq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
