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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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

// Fourth word of the raw buffer descriptors here: data format 32 bits (bits
// 15-18 = 4), no swizzle, no index stride, everything else zero.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Raw buffer descriptor over [base, base + bytes) as four words, for
// dma16_untracked: base address, no stride, `bytes` of range.  Loads at
// offsets outside the range (including "negative" offsets, which wrap past
// 2^31) return zeros.  Wave-uniform.
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3};
}

// 16 bytes per lane straight from a buffer into LDS: the wave's 64 lanes fill
// 1 KB at `lds_addr` in lane order (lane l at lds_addr + 16 l).  Written out
// as instructions, so that the compiler does not count it among its own
// memory operations.  The compiler treats a transposing LDS read
// as possibly overlapping any LDS write in flight from a buffer load and would
// otherwise wait for every tile load before each such read; here the caller's
// explicit vmcnt waits (before every barrier) are what order the tile loads
// against the reads.  The instruction writes no register (its destination is
// LDS), m0 is restored before the block ends, and the one wait state between
// the m0 write and its use is included.
__device__ __forceinline__ void dma16_untracked(u32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

// The same from a 64-bit global address per lane (used where the rows of a
// tile come from scattered cache blocks), written out for the same reason as
// dma16_untracked: no register written, m0 restored, the wait state included.
__device__ __forceinline__ void gdma16_untracked(const void* src, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// Transposing LDS reads through the compiler's builtins (the compiler waits
// for them before their results are used).
//  16-bit: within each 16 lanes, lane 4r+t names row r, columns 4t..4t+3;
//          lane c receives column c of the 4 rows.
//  8-bit:  within each 16 lanes, lane 2r+t names row r, bytes 8t..8t+7 of a
//          16-byte chunk; lane c receives byte c of that chunk from each of
//          the 8 rows (row r in byte r).
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t lds_addr) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (lds_i16x4*)(uintptr_t)lds_addr));
}
__device__ __forceinline__ u32x2 lds_read_tr8(uint32_t lds_addr) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                       (lds_i32x2*)(uintptr_t)lds_addr));
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
// The same for a wave-uniform count known only at run time (0..16).
__device__ __forceinline__ void wait_vm_lgkm0_rt(int vm) {
  switch (vm) {
    case 1: wait_vm_lgkm0<1>(); break;
    case 2: wait_vm_lgkm0<2>(); break;
    case 3: wait_vm_lgkm0<3>(); break;
    case 4: wait_vm_lgkm0<4>(); break;
    case 5: wait_vm_lgkm0<5>(); break;
    case 6: wait_vm_lgkm0<6>(); break;
    case 7: wait_vm_lgkm0<7>(); break;
    case 8: wait_vm_lgkm0<8>(); break;
    case 9: wait_vm_lgkm0<9>(); break;
    case 10: wait_vm_lgkm0<10>(); break;
    case 11: wait_vm_lgkm0<11>(); break;
    case 12: wait_vm_lgkm0<12>(); break;
    case 13: wait_vm_lgkm0<13>(); break;
    case 14: wait_vm_lgkm0<14>(); break;
    case 15: wait_vm_lgkm0<15>(); break;
    case 16: wait_vm_lgkm0<16>(); break;
    default: wait_vm_lgkm0<0>(); break;
  }
}

// A wave's 32 rows of output leave through LDS, so that every store
// instruction writes whole rows.  In the 32x32 accumulator layout lane l holds
// pieces of row l & 31, so one store straight from the accumulators would put
// 8 or 16 bytes into each of 32 rows.  Instead the wave writes its rows into
// kBytes of LDS of its own (16-byte chunks XOR-swizzled by row, so that
// neither these writes nor the row-wise reads meet bank conflicts), then
// reads them back kChunks lanes per row and stores kRowsPerRead whole rows per
// instruction.
template <int kRowBytes>
struct RowStage {
  static_assert(kRowBytes == 128 || kRowBytes == 256 || kRowBytes == 512, "row size");
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kRowsPerRead = 64 / kChunks;
  static constexpr int kReads = 32 / kRowsPerRead;
  static constexpr int kBytes = 32 * kRowBytes;
  // LDS byte offset of byte `col` (a multiple of 8) of row r.
  __device__ static __forceinline__ uint32_t at(int r, int col) {
    const int sw = kRowBytes == 128 ? (r >> 1) & 7 : r & 15;
    return (uint32_t)(r * kRowBytes + (((col >> 4) ^ sw) << 4) + (col & 15));
  }
  template <class V>
  __device__ static __forceinline__ void put(lds_char* ob, int r, int col, V v) {
    typedef __attribute__((address_space(3))) V lds_v;
    *(lds_v*)(ob + at(r, col)) = v;
  }
  // The wave's rows back from ob, this lane's share in x.  Only this wave
  // uses ob, so waiting for its own LDS writes is enough; the clobber keeps
  // the compiler from moving the reads above them.
  __device__ static __forceinline__ void read(const lds_char* ob, int lane, u32x4 (&x)[kReads]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int rr = lane / kChunks, cc = lane % kChunks;
#pragma unroll
    for (int i = 0; i < kReads; ++i)
      x[i] = *(const lds_u32x4*)(ob + at(i * kRowsPerRead + rr, cc * 16));
  }
  // x (from read) as rows of a buffer whose range ends at the last row to
  // write: exactly kReads store instructions, rows past the range dropped.
  __device__ static __forceinline__ void store_buf(const u32x4 (&x)[kReads], int lane,
                                                   __amdgpu_buffer_rsrc_t rsrc) {
    const int rr = lane / kChunks, cc = lane % kChunks;
#pragma unroll
    for (int i = 0; i < kReads; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(x[i], rsrc, (i * kRowsPerRead + rr) * kRowBytes + cc * 16,
                                             0, 0);
  }
  // Rows r < rows go to dst + r * stride (bytes).
  __device__ static __forceinline__ void store(const lds_char* ob, int lane, char* dst,
                                               size_t stride, int rows) {
    u32x4 x[kReads];
    read(ob, lane, x);
    const int rr = lane / kChunks, cc = lane % kChunks;
    char* const d0 = dst + cc * 16;
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      const int r = i * kRowsPerRead + rr;
      if (r < rows) *reinterpret_cast<u32x4*>(d0 + (size_t)r * stride) = x[i];
    }
  }
};

// Workgroup barrier without a memory fence: the caller has already waited for
// its own LDS traffic; the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace fa
