// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// log2(e): the kernels work with exp2 and fold log2(e) into the fp32 score scale.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite start for the running max (in scaled log2 units).  Masked scores are
// -inf, so exp2(-inf - kSentinel) = 0 and a fully masked tile leaves the state
// untouched instead of producing exp2(-inf - -inf) = NaN.
constexpr float kSentinel = -1.0e30f;

// ---------------------------------------------------------------------------
// 16-bit storage types.  Values travel as raw 16-bit patterns (uint16_t in
// memory, packed pairs in uint32_t registers).
// ---------------------------------------------------------------------------
struct BF16 {
  static __device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round two floats to nearest-even and pack (lo in bits 0..15).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
  // acc + lo(a)*lo(b) + hi(a)*hi(b) in one v_dot2_f32_bf16.
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
  }
  // acc + lo(x) + hi(x): a v_dot2 against (1, 1).
  static __device__ __forceinline__ float add_pair(uint32_t x, float acc) {
    return dot2(x, 0x3F803F80u, acc);
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
  }
  static __device__ __forceinline__ float add_pair(uint32_t x, float acc) {
    return dot2(x, 0x3C003C00u, acc);
  }
};

// The running max is raised lazily: only when a new tile's max exceeds it by
// more than kSlack (log2 units).  Until then weights exp2(s - m) stay below
// 2^kSlack = 256, which fp32 sums and bf16/fp16 operands hold comfortably, and
// the rescale of the history (a multiply per accumulator) is skipped.
constexpr float kSlack = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum of x over lanes l and l ^ 16 (v_permlane16_swap).
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// DPP lane moves within rows of 16 lanes (bound_ctrl: out-of-row reads give 0).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8 lanes
constexpr int kRowRor8 = 0x128;      // lane i <- lane (i+8) mod 16 within a row
constexpr int kRowMirror = 0x140;    // lane i <- lane 15-i within a row

// Sum / max over lanes l and l ^ 8 (a rotation by 8 inside each row of 16).
__device__ __forceinline__ float sum_xor8(float x) { return x + dpp<kRowRor8>(x); }
__device__ __forceinline__ float max_xor8(float x) { return fmaxf(x, dpp<kRowRor8>(x)); }

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  return x;
}
// Sum over each aligned group of 16 lanes (a DPP row).
__device__ __forceinline__ float sum16(float x) { return sum8(x) + dpp<kRowMirror>(sum8(x)); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Hardware hands consecutive workgroup ids to the 8 XCDs in turn.  Return a
// logical id such that each XCD receives one contiguous range of logical ids,
// so neighbouring tiles (which share K/V) meet in one XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int x = bid % kXcd, k = bid / kXcd;
  const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + k;
}

// Logical id of workgroup bid over total units laid out as groups of
// per_group consecutive units (a KV group: its query heads' Q tiles).  When
// the groups come in multiples of 8, XCD x takes groups x, x + 8, ... with
// each group's units back to back: units that share a group's K/V meet in
// one L2, and every XCD gets groups from every sequence of a ragged or paged
// batch (contiguous ranges would give each XCD a few whole sequences, and the
// longest would set the time).  Otherwise each XCD takes one contiguous range.
__device__ __forceinline__ int xcd_by_group(int bid, int total, int per_group) {
  if ((total / per_group) % 8 != 0) return xcd_contiguous(bid, total);
  const int x = bid % 8, k = bid / 8;
  return (x + 8 * (k / per_group)) * per_group + k % per_group;
}

// Causal form of xcd_by_group.  The units are (group, head of the group,
// Q-tile rank r); rank r = 0 is the heaviest (the last Q tile, which sees the
// most keys).  XCD x still takes the groups x, x + 8, ..., in chunks of up to
// four groups; within a chunk it hands out rank 0 of every unit first, then
// rank 1, and so on, so each chunk ends on its lightest tiles and no heavy
// tile starts last, while only a chunk's K/V (four groups) is live in the
// XCD's L2 at a time.  Returns the logical id (group * heads + head) *
// q_tiles + r, as xcd_by_group lays it out.
__device__ __forceinline__ int xcd_heavy_first(int bid, int total, int per_group, int q_tiles) {
  if ((total / per_group) % 8 != 0) return xcd_contiguous(bid, total);
  const int x = bid % 8, k = bid / 8;
  const int heads = per_group / q_tiles;  // query heads per group
  const int gx = total / per_group / 8;   // groups of XCD x
  const int cg = gx % 4 == 0 ? 4 : gx % 2 == 0 ? 2 : 1;  // groups per chunk
  const int per_chunk = cg * per_group;
  const int c = k / per_chunk, kk = k % per_chunk;
  const int r = kk / (cg * heads), j = kk % (cg * heads);
  const int gi = c * cg + j / heads, hg = j % heads;
  return ((x + 8 * gi) * heads + hg) * q_tiles + r;
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace fa
