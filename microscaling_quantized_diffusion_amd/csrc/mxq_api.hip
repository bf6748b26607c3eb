// Host side of the C ABI declared in include/mxq.h: argument validation,
// workspace layout and kernel dispatch.  Every check runs before anything is
// enqueued, so a failing call launches nothing.
#include <mutex>
#include <string.h>

#include "mxq_internal.h"

using namespace mxq;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* a, const void* b) { return (((uintptr_t)a | (uintptr_t)b) & 3u) == 0; }

int block_of(mxq_format fmt) { return fmt == MXQ_FMT_NVFP4 ? 16 : 32; }

bool valid_format(mxq_format fmt) {
  return fmt == MXQ_FMT_MXFP8 || fmt == MXQ_FMT_MXFP4 || fmt == MXQ_FMT_NVFP4 || fmt == MXQ_FMT_MXFP6_E2M3 ||
         fmt == MXQ_FMT_MXFP6_E3M2;
}
bool is_fp6(mxq_format fmt) { return fmt == MXQ_FMT_MXFP6_E2M3 || fmt == MXQ_FMT_MXFP6_E3M2; }

// A format argument is a base format, optionally OR-ed with MXQ_SCALE_RCEIL
// and MXQ_SCALES_PACKED (MX formats only).  Splits it; false for anything
// else.  Each entry point decides what the packed flag means for it.
bool split_format(mxq_format arg, mxq_format* base, int* rceil, int* packed) {
  const int v = (int)arg;
  *base = (mxq_format)(v & 0xFF);
  *rceil = (v & MXQ_SCALE_RCEIL) ? 1 : 0;
  *packed = (v & MXQ_SCALES_PACKED) ? 1 : 0;
  if ((v & ~0xFF & ~MXQ_SCALE_RCEIL & ~MXQ_SCALES_PACKED) != 0 || !valid_format(*base)) return false;
  return !((*rceil || *packed) && *base == MXQ_FMT_NVFP4);
}
bool split_format(mxq_format arg, mxq_format* base, int* rceil) {
  int packed = 0;
  return split_format(arg, base, rceil, &packed) && !packed;
}

// K must be a positive multiple of the block; sizes must fit the kernels'
// 32-bit row/column indices.
bool valid_k(mxq_format fmt, int64_t K) { return K > 0 && K % block_of(fmt) == 0 && K <= (1 << 30); }
bool valid_dim(int64_t d) { return d >= 0 && d <= (int64_t)1 << 30; }
// GEMM limits: the kernels address a tile's rows (up to 256 rows of K codes,
// or 2K bytes of bf16) through one 32-bit buffer range with 32-bit lane
// offsets, and launch one workgroup per tile (down to 128 x 128 outputs).
constexpr int64_t kGemmMaxK = (int64_t)1 << 22;
constexpr int64_t kGemmMaxMN = (int64_t)1 << 39;
bool valid_gemm(int64_t M, int64_t N, int64_t K) {
  return valid_dim(M) && valid_dim(N) && K <= kGemmMaxK && M * N <= kGemmMaxMN;
}

size_t code_bytes(mxq_format fmt, int64_t rows, int64_t K) {
  return (size_t)rows * (size_t)(fmt == MXQ_FMT_MXFP8 || is_fp6(fmt) ? K : K / 2);
}
size_t scale_bytes(mxq_format fmt, int64_t rows, int64_t K) { return (size_t)rows * (size_t)(K / block_of(fmt)); }
// The packed scale layout: whole K stages of the MX GEMM (128 elements of
// FP8 / FP6, 256 of FP4), rows padded to whole groups of 32, and a block
// count the quantizer indexes in 32 bits.
int64_t stage_k(mxq_format fmt) { return fmt == MXQ_FMT_MXFP4 ? 256 : 128; }
int64_t padded_rows(int64_t rows) { return (rows + 31) / 32 * 32; }
bool packable(mxq_format fmt, int64_t rows, int64_t K) {
  return fmt != MXQ_FMT_NVFP4 && K % stage_k(fmt) == 0 && padded_rows(rows) * (K / 32) < ((int64_t)1 << 32);
}
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Fused workspace: [A codes | A scales | tensor scale (NVFP4) | amax partials (NVFP4)],
// each section 256-byte aligned.
struct FusedLayout {
  size_t codes, scales, ts, partials, total;
};
FusedLayout fused_layout(mxq_format fmt, int64_t M, int64_t K) {
  FusedLayout L{};
  L.codes = 0;
  L.scales = round256(code_bytes(fmt, M, K));
  // MX scales sized for padded rows, so the packed layout fits too
  L.ts = L.scales + round256(scale_bytes(fmt, fmt == MXQ_FMT_NVFP4 ? M : padded_rows(M), K));
  L.partials = L.ts + (fmt == MXQ_FMT_NVFP4 ? 256 : 0);
  L.total = L.partials + (fmt == MXQ_FMT_NVFP4 ? round256((size_t)nvfp4_partials_count(M * K) * 4) : 0);
  return L;
}

mxq_status launch_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_LAUNCH; }

// The fixed scratch of mxq_quant_gemm_fused_noalloc: one copy per GPU, in
// the code object's zero-initialised data (nothing is allocated at run
// time).  In host code `scratch` names a host-side stand-in, not the device
// array: kernels get the address from hipGetSymbolAddress, looked up once
// per device with that device current.
__device__ __align__(256) uint8_t scratch[MXQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or nullptr if it
// cannot be found (no current device, or the lookup failed).
uint8_t* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = (uint8_t*)ptr;
  }
  return g_scratch_ptr[dev];
}

// element format of an MX format: 1 = E4M3, 2 = E2M1, 3 = E2M3, 4 = E3M2
int elem_of(mxq_format fmt) {
  return fmt == MXQ_FMT_MXFP8 ? 1 : fmt == MXQ_FMT_MXFP6_E2M3 ? 3 : fmt == MXQ_FMT_MXFP6_E3M2 ? 4 : 2;
}

}  // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_FORMAT: return "unknown format";
    case MXQ_ERR_SHAPE: return "invalid shape (negative size, or K not a positive multiple of the block)";
    case MXQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MXQ_ERR_UNSUPPORTED: return "unsupported request";
    case MXQ_ERR_LAUNCH: return "kernel launch failed";
    case MXQ_ERR_TOO_LARGE: return "problem larger than the library's fixed scratch (MXQ_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int mxq_should_quantize(int64_t M, int64_t K, int64_t N) {
  int64_t mn = M < K ? M : K;
  mn = mn < N ? mn : N;
  return mn >= 1024 ? 1 : 0;
}

size_t mxq_workspace_bytes(mxq_format fmt_arg, int64_t M, int64_t K, int fused) {
  mxq_format fmt;
  int rceil, packed;  // neither changes the workspace
  if (!split_format(fmt_arg, &fmt, &rceil, &packed) || !valid_dim(M) || !valid_k(fmt, K)) return 0;
  if (fused) return fused_layout(fmt, M, K).total;
  if (fmt == MXQ_FMT_NVFP4) return round256((size_t)nvfp4_partials_count(M * K) * 4);
  return 0;
}

mxq_status mxq_quantize(mxq_format fmt_arg, const void* x_bf16, int64_t rows, int64_t cols, void* codes,
                        void* scales, float* tensor_scale, void* workspace, size_t workspace_bytes, void* stream) {
  mxq_format fmt;
  int rceil, packed;
  if (!split_format(fmt_arg, &fmt, &rceil, &packed)) return MXQ_ERR_FORMAT;
  if (!valid_dim(rows) || !valid_k(fmt, cols)) return MXQ_ERR_SHAPE;
  if (packed && !packable(fmt, rows, cols)) return MXQ_ERR_UNSUPPORTED;
  if (rows == 0) return MXQ_OK;  // nothing to read or write, whatever the pointers
  if (!x_bf16 || !codes || !scales) return MXQ_ERR_NULL;
  if (fmt == MXQ_FMT_NVFP4 && !tensor_scale) return MXQ_ERR_NULL;
  if (fmt != MXQ_FMT_NVFP4 && tensor_scale) return MXQ_ERR_UNSUPPORTED;
  if (!aligned16(x_bf16) || !aligned16(codes)) return MXQ_ERR_ALIGN;
  const size_t need = mxq_workspace_bytes(fmt, rows, cols, 0);
  if (need && (!workspace || workspace_bytes < need)) return MXQ_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return MXQ_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (fmt == MXQ_FMT_NVFP4)
    return launch_status(launch_nvfp4_quant((const uint16_t*)x_bf16, rows, cols, (uint8_t*)codes, (uint8_t*)scales,
                                            tensor_scale, (uint32_t*)workspace, s));
  return launch_status(launch_mx_quant(elem_of(fmt), rceil, packed, (const uint16_t*)x_bf16, rows, cols,
                                       (uint8_t*)codes, (uint8_t*)scales, s));
}

mxq_status mxq_gemm(mxq_format fmt_arg, int64_t M, int64_t N, int64_t K, const void* a_codes, const void* a_scales,
                    const float* a_tensor_scale, const void* w_codes, const void* w_scales,
                    const float* w_tensor_scale, const void* bias_bf16, void* out_bf16, void* stream) {
  mxq_format fmt;
  int rceil, packed;  // quantizes nothing: the scale rule does not apply
  if (!split_format(fmt_arg, &fmt, &rceil, &packed)) return MXQ_ERR_FORMAT;
  if (!valid_k(fmt, K) || !valid_gemm(M, N, K)) return MXQ_ERR_SHAPE;
  if (packed && K % stage_k(fmt) != 0) return MXQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return MXQ_OK;  // empty output: nothing to launch, whatever the pointers
  if (!a_codes || !a_scales || !w_codes || !w_scales || !out_bf16) return MXQ_ERR_NULL;
  if (fmt == MXQ_FMT_NVFP4 && (!a_tensor_scale || !w_tensor_scale)) return MXQ_ERR_NULL;
  if (fmt != MXQ_FMT_NVFP4 && (a_tensor_scale || w_tensor_scale)) return MXQ_ERR_UNSUPPORTED;
  if (!aligned16(a_codes) || !aligned16(w_codes) || !aligned16(out_bf16)) return MXQ_ERR_ALIGN;
  if (is_fp6(fmt) && K % 128 != 0) return MXQ_ERR_UNSUPPORTED;
  if ((is_fp6(fmt) || packed) && !aligned4(a_scales, w_scales)) return MXQ_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (fmt == MXQ_FMT_NVFP4)
    return launch_status(launch_nvfp4_gemm(M, N, K, (const uint8_t*)a_codes, (const uint8_t*)a_scales, a_tensor_scale,
                                           (const uint8_t*)w_codes, (const uint8_t*)w_scales, w_tensor_scale,
                                           (const uint16_t*)bias_bf16, (uint16_t*)out_bf16, s));
  return launch_status(launch_mx_gemm(elem_of(fmt), packed, M, N, K, (const uint8_t*)a_codes,
                                      (const uint8_t*)a_scales, (const uint8_t*)w_codes, (const uint8_t*)w_scales,
                                      (const uint16_t*)bias_bf16, (uint16_t*)out_bf16, s));
}

}  // extern "C"

namespace {
// mxq_quant_gemm_fused's checks and launches with the workspace given by
// `get_ws`, which is called only once every argument check has passed; it
// returns the workspace pointer and its size, or a status to return.
template <typename GetWs>
mxq_status fused_call(mxq_format fmt_arg, int64_t M, int64_t N, int64_t K, const void* a_bf16, const void* w_codes,
                      const void* w_scales, const float* w_tensor_scale, const void* bias_bf16, void* out_bf16,
                      void* stream, GetWs get_ws) {
  mxq_format fmt;
  int rceil, packed;  // packed: W's scales are packed, and A's are written packed into the workspace
  if (!split_format(fmt_arg, &fmt, &rceil, &packed)) return MXQ_ERR_FORMAT;
  if (!valid_k(fmt, K) || !valid_gemm(M, N, K)) return MXQ_ERR_SHAPE;
  if (packed && !packable(fmt, M, K)) return MXQ_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return MXQ_OK;  // empty output: nothing to launch, whatever the pointers
  if (!a_bf16 || !w_codes || !w_scales || !out_bf16) return MXQ_ERR_NULL;
  if (fmt == MXQ_FMT_NVFP4 && !w_tensor_scale) return MXQ_ERR_NULL;
  if (fmt != MXQ_FMT_NVFP4 && w_tensor_scale) return MXQ_ERR_UNSUPPORTED;
  if (!aligned16(a_bf16) || !aligned16(w_codes) || !aligned16(out_bf16)) return MXQ_ERR_ALIGN;
  if (is_fp6(fmt) && K % 128 != 0) return MXQ_ERR_UNSUPPORTED;
  // the activation scales are in the workspace (256-byte aligned)
  if ((is_fp6(fmt) || packed) && !aligned4(w_scales, w_scales)) return MXQ_ERR_ALIGN;
  const FusedLayout L = fused_layout(fmt, M, K);
  uint8_t* ws = nullptr;
  const mxq_status wst = get_ws(L.total, &ws);
  if (wst != MXQ_OK) return wst;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* a_codes = ws + L.codes;
  uint8_t* a_scales = ws + L.scales;
  hipError_t e;
  if (fmt == MXQ_FMT_NVFP4) {
    float* a_ts = (float*)(ws + L.ts);
    e = launch_nvfp4_quant((const uint16_t*)a_bf16, M, K, a_codes, a_scales, a_ts, (uint32_t*)(ws + L.partials), s);
    if (e != hipSuccess) return MXQ_ERR_LAUNCH;
    e = launch_nvfp4_gemm(M, N, K, a_codes, a_scales, a_ts, (const uint8_t*)w_codes, (const uint8_t*)w_scales,
                          w_tensor_scale, (const uint16_t*)bias_bf16, (uint16_t*)out_bf16, s);
    return launch_status(e);
  }
  e = launch_mx_quant(elem_of(fmt), rceil, packed, (const uint16_t*)a_bf16, M, K, a_codes, a_scales, s);
  if (e != hipSuccess) return MXQ_ERR_LAUNCH;
  e = launch_mx_gemm(elem_of(fmt), packed, M, N, K, a_codes, a_scales, (const uint8_t*)w_codes,
                     (const uint8_t*)w_scales, (const uint16_t*)bias_bf16, (uint16_t*)out_bf16, s);
  return launch_status(e);
}
}  // namespace

extern "C" {

mxq_status mxq_quant_gemm_fused(mxq_format fmt_arg, int64_t M, int64_t N, int64_t K, const void* a_bf16,
                                const void* w_codes, const void* w_scales, const float* w_tensor_scale,
                                const void* bias_bf16, void* out_bf16, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return fused_call(fmt_arg, M, N, K, a_bf16, w_codes, w_scales, w_tensor_scale, bias_bf16, out_bf16, stream,
                    [&](size_t need, uint8_t** ws) {
                      if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
                      if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
                      *ws = (uint8_t*)workspace;
                      return MXQ_OK;
                    });
}

mxq_status mxq_quant_gemm_fused_noalloc(mxq_format fmt_arg, int64_t M, int64_t N, int64_t K, const void* a_bf16,
                                        const void* w_codes, const void* w_scales, const float* w_tensor_scale,
                                        const void* bias_bf16, void* out_bf16, void* stream) {
  return fused_call(fmt_arg, M, N, K, a_bf16, w_codes, w_scales, w_tensor_scale, bias_bf16, out_bf16, stream,
                    [&](size_t need, uint8_t** ws) {
                      if (need > MXQ_NOALLOC_SCRATCH_BYTES) return MXQ_ERR_TOO_LARGE;
                      *ws = device_scratch();
                      return *ws ? MXQ_OK : MXQ_ERR_LAUNCH;
                    });
}

namespace {
// Row strides of a quantized output (bytes; 0 = dense): the codes' a multiple
// of 16 (16-byte row stores) and at least a dense row, the scales' at least
// a dense row.
mxq_status check_out_strides(int elem, int64_t cols, int64_t codes_ld, int64_t scales_ld) {
  const int64_t dense = elem == 1 ? cols : cols / 2;
  if (codes_ld < 0 || scales_ld < 0 || (codes_ld && codes_ld < dense) || (scales_ld && scales_ld < cols / 32))
    return MXQ_ERR_SHAPE;
  if (codes_ld % 16 != 0) return MXQ_ERR_ALIGN;
  return MXQ_OK;
}
}  // namespace

mxq_status mxq_gemm_requant(mxq_format fmt_arg, int64_t M, int64_t N, int64_t K, const void* a_codes,
                            const void* a_scales, const void* w_codes, const void* w_scales, const void* bias_bf16,
                            int act, mxq_format out_fmt_arg, void* out_bf16, void* out_codes, void* out_scales,
                            int64_t out_codes_ld, int64_t out_scales_ld, void* stream) {
  mxq_format fmt, out_fmt;
  int in_rceil, rceil;  // the input operands are already quantized: only out_fmt's rule applies
  if (!split_format(fmt_arg, &fmt, &in_rceil) || !split_format(out_fmt_arg, &out_fmt, &rceil))
    return MXQ_ERR_FORMAT;
  if (!valid_k(fmt, K) || !valid_gemm(M, N, K) || N % 32 != 0) return MXQ_ERR_SHAPE;
  const mxq_status st = check_out_strides(elem_of(out_fmt), N, out_codes_ld, out_scales_ld);
  if (st == MXQ_ERR_SHAPE) return st;
  if (M == 0 || N == 0) return MXQ_OK;  // empty output: nothing to launch, whatever the pointers
  if (!a_codes || !a_scales || !w_codes || !w_scales || !out_codes || !out_scales) return MXQ_ERR_NULL;
  if (st != MXQ_OK || !aligned16(a_codes) || !aligned16(w_codes) || !aligned16(out_codes)) return MXQ_ERR_ALIGN;
  if (out_bf16 && !aligned16(out_bf16)) return MXQ_ERR_ALIGN;
  // operands MXFP8 / MXFP6 / MXFP4; outputs MXFP8 / MXFP4
  if (fmt == MXQ_FMT_NVFP4 || out_fmt == MXQ_FMT_NVFP4 || is_fp6(out_fmt) || (act != 0 && act != 1))
    return MXQ_ERR_UNSUPPORTED;
  if (!mx_requant_supported(elem_of(fmt), N, K, (const uint8_t*)a_scales, (const uint8_t*)w_scales))
    return MXQ_ERR_UNSUPPORTED;
  return launch_status(launch_mx_gemm_requant(elem_of(fmt), elem_of(out_fmt), rceil, act, M, N, K,
                                              (const uint8_t*)a_codes,
                                              (const uint8_t*)a_scales, (const uint8_t*)w_codes,
                                              (const uint8_t*)w_scales, (const uint16_t*)bias_bf16,
                                              (uint16_t*)out_bf16, (uint8_t*)out_codes, (uint8_t*)out_scales,
                                              out_codes_ld, out_scales_ld, (hipStream_t)stream));
}

namespace {
constexpr int64_t kAttnHeadDim = 128;
constexpr int64_t kAttnMaxBH = 65535;         // one grid row per (batch, head)
constexpr int64_t kAttnMaxS = (int64_t)1 << 24;
// shape status of an attention call: sizes, then what this build implements
mxq_status attention_shape(int64_t B, int64_t H, int64_t S, int64_t D) {
  if (B < 0 || H < 0 || S < 0 || D <= 0 || S > kAttnMaxS || (B > 0 && H > kAttnMaxBH / B)) return MXQ_ERR_SHAPE;
  if (D != kAttnHeadDim || S % 64 != 0) return MXQ_ERR_UNSUPPORTED;
  return MXQ_OK;
}
}  // namespace

size_t mxq_attention_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D) {
  if (attention_shape(B, H, S, D) != MXQ_OK) return 0;
  return attention_layout(B * H, S).total;
}

mxq_status mxq_attention_fp8(int64_t B, int64_t H, int64_t S, int64_t D, const void* q_bf16, const void* k_bf16,
                             const void* v_bf16, void* out_bf16, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const mxq_status sh = attention_shape(B, H, S, D);
  if (sh == MXQ_ERR_SHAPE) return sh;
  if (B * H == 0 || S == 0) return MXQ_OK;  // empty: nothing to launch, whatever the pointers
  if (sh != MXQ_OK) return sh;
  if (!q_bf16 || !k_bf16 || !v_bf16 || !out_bf16) return MXQ_ERR_NULL;
  if (!aligned16(q_bf16) || !aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(out_bf16)) return MXQ_ERR_ALIGN;
  const size_t need = attention_layout(B * H, S).total;
  if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
  return launch_status(launch_attention_fp8(B * H, S, (const uint16_t*)q_bf16, (const uint16_t*)k_bf16,
                                            (const uint16_t*)v_bf16, (uint16_t*)out_bf16, (uint8_t*)workspace,
                                            (hipStream_t)stream));
}

mxq_status mxq_attention_fp8_requant(int64_t B, int64_t H, int64_t S, int64_t D, const void* q_bf16,
                                     const void* k_bf16, const void* v_bf16, mxq_format out_fmt_arg,
                                     void* out_codes, void* out_scales, int64_t out_codes_ld,
                                     int64_t out_scales_ld, void* workspace, size_t workspace_bytes, void* stream) {
  mxq_format out_fmt;
  int rceil;
  if (!split_format(out_fmt_arg, &out_fmt, &rceil)) return MXQ_ERR_FORMAT;
  const mxq_status sh = attention_shape(B, H, S, D);
  if (sh == MXQ_ERR_SHAPE) return sh;
  const mxq_status st = check_out_strides(elem_of(out_fmt), H * D, out_codes_ld, out_scales_ld);
  if (st == MXQ_ERR_SHAPE) return st;
  if (B * H == 0 || S == 0) return MXQ_OK;  // empty: nothing to launch, whatever the pointers
  if (sh != MXQ_OK || out_fmt == MXQ_FMT_NVFP4 || is_fp6(out_fmt)) return MXQ_ERR_UNSUPPORTED;
  if (!q_bf16 || !k_bf16 || !v_bf16 || !out_codes || !out_scales) return MXQ_ERR_NULL;
  if (st != MXQ_OK || !aligned16(q_bf16) || !aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(out_codes))
    return MXQ_ERR_ALIGN;
  const size_t need = attention_layout(B * H, S).total;
  if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
  const int elem = elem_of(out_fmt);
  const int64_t qld = out_codes_ld ? out_codes_ld : (elem == 1 ? H * D : H * D / 2);
  const int64_t sld = out_scales_ld ? out_scales_ld : H * D / 32;
  return launch_status(launch_attention_fp8(B * H, S, (const uint16_t*)q_bf16, (const uint16_t*)k_bf16,
                                            (const uint16_t*)v_bf16, nullptr, (uint8_t*)workspace,
                                            (hipStream_t)stream, elem, rceil, H, (uint8_t*)out_codes,
                                            (uint8_t*)out_scales, qld, sld));
}

mxq_status mxq_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* a_bf16, const void* w_bf16,
                         const void* bias_bf16, void* out_bf16, void* stream) {
  if (K <= 0 || !valid_gemm(M, N, K)) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;  // empty output: nothing to launch, whatever the pointers
  if (!a_bf16 || !w_bf16 || !out_bf16) return MXQ_ERR_NULL;
  if (!aligned16(a_bf16) || !aligned16(w_bf16) || !aligned16(out_bf16)) return MXQ_ERR_ALIGN;
  return launch_status(launch_bf16_gemm(M, N, K, (const uint16_t*)a_bf16, (const uint16_t*)w_bf16,
                                        (const uint16_t*)bias_bf16, (uint16_t*)out_bf16, (hipStream_t)stream));
}

}  // extern "C"
