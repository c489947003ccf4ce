// Merge of attention pieces computed over disjoint key ranges.
//
// A piece s holds, per query row, the output normalised over its own keys
// (o_s) and the natural log of its softmax denominator (lse_s = m_s + ln l_s).
// The whole-range result is the rescale the online-softmax recurrence applies
// between tiles, applied once to whole pieces (llminference.xinbetween.com
// S12, "除了快，它还解锁了什么" and exercise 1): with L = max_s lse_s and
// w_s = exp(lse_s - L), O = sum_s w_s o_s / sum_s w_s and lse = L + ln sum_s w_s.
// Pieces with lse_s = -inf (no key of the row in that range) weigh nothing,
// and a row that no piece covers gives O = 0, lse = -inf.
//
// One thread per 4 adjacent columns of a row (16-byte loads of every piece);
// a workgroup covers 256 / (dv / 4) consecutive rows.  The pass is bandwidth
// bound (it reads every piece once) and runs on the vector ALUs.  The pieces
// are read four at a time with all their loads in flight together, o with
// nontemporal loads (read once); a piece without keys is left out by a
// select, so its o never reaches the sum whatever it holds.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int kMergeThreads = 256;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

template <int OUT>  // output type: 0 float32, 1 float16, 2 bfloat16
__global__ __launch_bounds__(kMergeThreads) void fa_merge_lse(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int parts,
    long long rows, int dv, int rows_per_wg, void* __restrict__ o, float* __restrict__ lse_out) {
  const int quads = dv / 4;  // threads per row
  const int r_local = threadIdx.x / quads;
  if (r_local >= rows_per_wg) return;
  const long long row = (long long)blockIdx.x * rows_per_wg + r_local;
  if (row >= rows) return;
  const int c = (threadIdx.x - r_local * quads) * 4;

  const float* lse_row = lse_parts + row;
  const float* o_row = o_parts + (size_t)row * dv + c;
  const size_t o_step = (size_t)rows * dv;
  float L = -__builtin_inff();
  for (int s = 0; s < parts; ++s) L = fmaxf(L, lse_row[(size_t)s * rows]);
  const bool has = L > -__builtin_inff();
  float W = 0.f;
  float4 a = {0.f, 0.f, 0.f, 0.f};
  constexpr int kBatch = 4;
  for (int s0 = 0; s0 < parts; s0 += kBatch) {
    float ls[kBatch];
    f32x4 x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < parts) {  // uniform across the grid
        ls[u] = lse_row[(size_t)(s0 + u) * rows];
        x[u] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(o_row + (size_t)(s0 + u) * o_step));
      } else {
        ls[u] = -__builtin_inff();
        x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // a piece without keys weighs nothing and its o is not used
      const bool ok = has && ls[u] > -__builtin_inff();
      const float w = ok ? expf(ls[u] - L) : 0.f;
      W += w;
      a.x = ok ? fmaf(w, x[u][0], a.x) : a.x;
      a.y = ok ? fmaf(w, x[u][1], a.y) : a.y;
      a.z = ok ? fmaf(w, x[u][2], a.z) : a.z;
      a.w = ok ? fmaf(w, x[u][3], a.w) : a.w;
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  a.x *= inv;
  a.y *= inv;
  a.z *= inv;
  a.w *= inv;
  const size_t off = (size_t)row * dv + c;
  if constexpr (OUT == 0) {
    *reinterpret_cast<float4*>(static_cast<float*>(o) + off) = a;
  } else if constexpr (OUT == 1) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + off) =
        u32x2{F16::pack(a.x, a.y), F16::pack(a.z, a.w)};
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + off) =
        u32x2{BF16::pack(a.x, a.y), BF16::pack(a.z, a.w)};
  }
  if (lse_out && c == 0) lse_out[row] = has ? L + logf(W) : -__builtin_inff();
}

hipError_t launch_merge(const MergeArgs& a) {
  const int rows_per_wg = kMergeThreads / (a.dv / 4);
  const long long wgs = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)wgs), block(kMergeThreads);
  hipStream_t st = (hipStream_t)a.stream;
  if (a.out_dtype == 0)
    hipLaunchKernelGGL(fa_merge_lse<0>, grid, block, 0, st, a.o_parts, a.lse_parts, a.parts,
                       a.rows, a.dv, rows_per_wg, a.o, a.lse_out);
  else if (a.out_dtype == 1)
    hipLaunchKernelGGL(fa_merge_lse<1>, grid, block, 0, st, a.o_parts, a.lse_parts, a.parts,
                       a.rows, a.dv, rows_per_wg, a.o, a.lse_out);
  else
    hipLaunchKernelGGL(fa_merge_lse<2>, grid, block, 0, st, a.o_parts, a.lse_parts, a.parts,
                       a.rows, a.dv, rows_per_wg, a.o, a.lse_out);
  return hipGetLastError();
}

}  // namespace fa
