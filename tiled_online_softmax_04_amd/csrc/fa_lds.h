// LDS staging helpers shared by the gfx950 prefill kernels: buffer loads that
// write LDS directly, wait-count and barrier primitives, and the K-row
// permutation that lines the score accumulator up with the P.V operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"

namespace fa {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// Row placement of the K tile inside each 32-row block.  The accumulator of a
// 32x32 MFMA (any input type) gives lane l, element i the row
// 8*(i/4) + 4*(l/32) + (i%4).  Storing key r at LDS row kappa(r) (swap rows
// 4..7 with 8..11 and 20..23 with 24..27) makes element i of lane l hold key
// 16*(i/8) + 8*(l/32) + (i%8): runs of eight consecutive keys per half-wave,
// which is the B-operand layout of the P.V MFMA and what one transposing LDS
// read of V delivers.  kappa is its own inverse.
__device__ __forceinline__ int kappa(int r) {
  return r ^ ((((r >> 2) ^ (r >> 3)) & 1) * 0xC);
}

// Raw buffer descriptor over [base, base + bytes).  Loads at offsets outside
// the range (including "negative" offsets, which wrap past 2^31) return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane straight from a buffer into LDS: the wave's 64 lanes fill
// 1 KB at `lds_base` in lane order (lane l at lds_base + 16*l).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, lds_char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// The same from a 64-bit global address per lane (used where the rows of a
// tile come from scattered cache blocks).
__device__ __forceinline__ void gdma16(const void* src, lds_char* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

// s_waitcnt lgkmcnt(0) (vmcnt, expcnt untouched).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Make x look redefined here, so no use of x is scheduled above this point.
template <class X>
__device__ __forceinline__ void reg_barrier(X& x) {
  asm volatile("" : "+v"(x));
}

// s_waitcnt with vmcnt <= VM and lgkmcnt == 0 (expcnt untouched).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without a memory fence: the caller has already waited for
// its own LDS traffic; the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace fa
