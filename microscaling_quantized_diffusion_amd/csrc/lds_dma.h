// Buffer-resource loads straight into LDS (LDS DMA) and the wait-count
// helpers that go with them, shared by the GEMM and attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Buffer resource over a tile's rows: loads at offsets >= num_records return
// zeros, which pads rows beyond M / N and the K tail with zero codes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;

// LDS DMA of `bytes` per lane (lane i lands at lds + i * bytes) from byte
// voff + soff of the buffer; voff is the per-lane part, soff a wave-uniform
// one (the instruction's scalar offset), so that a loop-invariant voff needs
// no temporary register whose reuse would force a wait on the DMA.  Kept as
// plain device functions: the builtin inside a generic lambda fails the host
// pass's substitution and drops the kernel's launch stub.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}
// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Issued through
// the builtin rather than inline asm so that the compiler's own wait
// bookkeeping sees it; an asm wait is invisible to it, and it then re-waits
// on DMA that was issued after the asm wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (0x7 << 4)); }

}  // namespace mxq
