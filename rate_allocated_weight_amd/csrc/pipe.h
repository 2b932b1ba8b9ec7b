// Helpers of the global -> LDS operand rings used by the MFMA kernels (int8 interference
// product, Y = W U^T, covariance). Operands are moved by global_load_lds_dwordx4 (each
// instruction of a wave fills 1 KiB of LDS, lane l at byte 16 l); a ring of S buffers keeps
// S - 1 K-steps in flight. The vector-memory counter counts those loads in issue order, so
// "step t has landed" is "at most (steps issued after t) x (loads per step) still pending".
#pragma once

#include <hip/hip_runtime.h>

namespace wsic {
namespace pipe {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const char lds_char;

// Workgroup barrier without the memory fence of __syncthreads(): that fence would also wait
// for every operand load still in flight. This wave's LDS traffic is drained first; the DMA
// writes a wave depends on are ordered by wait_vm before it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most `ahead` steps of PER loads each are pending (ahead in [0, MAXA])
template <int PER, int MAXA>
__device__ __forceinline__ void wait_ahead(int ahead) {
  static_assert(MAXA >= 0 && MAXA <= 4, "ring depth");
  (void)ahead;
  if (MAXA >= 4 && ahead >= 4) wait_vm<PER * (MAXA >= 4 ? 4 : 0)>();
  else if (MAXA >= 3 && ahead == 3) wait_vm<PER * (MAXA >= 3 ? 3 : 0)>();
  else if (MAXA >= 2 && ahead == 2) wait_vm<PER * (MAXA >= 2 ? 2 : 0)>();
  else if (MAXA >= 1 && ahead == 1) wait_vm<PER * (MAXA >= 1 ? 1 : 0)>();
  else wait_vm<0>();
}

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

// The same through a buffer resource: an offset at or past `bytes` reads zeros (the range check
// of raw buffer loads, checked on gfx950), so edges need no branch and no zero page.
constexpr unsigned OUT_OF_RANGE = 0x7FFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, 0, 0, 0);
}

}  // namespace pipe
}  // namespace wsic
