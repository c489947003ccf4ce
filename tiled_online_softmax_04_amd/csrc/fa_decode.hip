// Paged grouped-query decode for gfx950: split-K partial pass + merge pass.
//
// One query token per sequence.  The keys of a sequence live in a paged cache
// reached through its block table (the S12 chapter's paged loop, "实现"); the
// query heads of one group share a KV head and read each K/V row once
// ("它如何与你已经搭好的部分组合").  Decode has a single query row, so the
// parallelism comes from the keys instead (flash-decoding, S12): the key range
// of a sequence is cut into splits, each split runs the online-softmax
// recurrence in its own workgroup and leaves a partial (m, l, acc), and a second
// kernel merges the partials with the same rescale (S12 exercise 1).
//
// This pass moves about 4 FLOP per byte, far below the MFMA ridge point, so it
// is bandwidth bound: the kernel streams K/V with 16-byte loads straight into
// VGPRs and does the arithmetic on the vector ALUs.
//
// Lane layout of the split kernel: a wave takes 16 consecutive tokens at a
// time; lane = 8 * slot + sub, token slot `slot` (0..7) handles tokens slot and
// slot + 8 of the chunk, and `sub` (0..7) handles the 16-byte chunks sub and
// sub + 8 of each row (D = 128; D = 64 has one chunk per lane).  A dot product
// is finished by a sum over the 8 lanes of a slot (DPP).  The running max of a
// head is kept uniform across the wave, so the rescale of the history is a
// wave-uniform branch taken only when the max moves.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecChunk = 16;  // tokens per wave step

template <class T, int D, int GW>
__global__ __launch_bounds__(kDecThreads) void fa_decode_split(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int bs, int Hq, int Hkv, int group, int subgroups,
    int maxb, int num_blocks, int split_tokens, int max_splits, float c,
    float* __restrict__ part_m,
    float* __restrict__ part_l, float* __restrict__ part_acc) {
  constexpr int NCH = D / 64;     // 16-byte chunks per lane per row
  constexpr int NE = NCH * 8;     // elements per lane per row
  __shared__ float red_m[kDecWaves][GW];
  __shared__ float red_l[kDecWaves][GW];
  __shared__ float red_acc[kDecWaves][GW][D];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / subgroups;
  const int sg = blockIdx.y % subgroups;
  const int seq = blockIdx.z;
  const int L = seq_lens[seq];
  const int tok0 = split * split_tokens;
  if (tok0 >= L) return;  // empty split: the merge never reads it
  const int tok1 = min(L, tok0 + split_tokens);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int slot = lane >> 3, sub = lane & 7;
  const int h0 = kvh * group + sg * GW;  // first query head of this workgroup

  // Query values at this lane's dims, float32.
  float qf[GW][NE];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    const uint16_t* qh = Q + ((size_t)seq * Hq + h0 + g) * D;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const u32x4 x = load16(qh + (sub + 8 * cc) * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[g][cc * 8 + 2 * e] = T::lo(x[e]);
        qf[g][cc * 8 + 2 * e + 1] = T::hi(x[e]);
      }
    }
  }

  float m_run[GW], l_run[GW], acc[GW][NE];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m_run[g] = kSentinel;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[g][e] = 0.f;
  }

  const int32_t* bt = block_table + (size_t)seq * maxb;
  const size_t row_stride = (size_t)Hkv * D;

  for (int t0 = tok0 + w * kDecChunk; t0 < tok1; t0 += kDecWaves * kDecChunk) {
    u32x4 kx[2][NCH], vx[2][NCH];
    bool valid[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = t0 + slot + 8 * tt;
      valid[tt] = tok < tok1;
      const int tk = valid[tt] ? tok : tok0;
      // Table entries and lengths outside their stated ranges are clamped so
      // that no access leaves the buffers (the result is then unspecified).
      const int phys = min(max(bt[min(tk / bs, maxb - 1)], 0), num_blocks - 1);
      const size_t row = ((size_t)phys * bs + (tk % bs)) * row_stride + (size_t)kvh * D;
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        kx[tt][cc] = valid[tt] ? load16(Kc + row + (sub + 8 * cc) * 8) : u32x4{0, 0, 0, 0};
        vx[tt][cc] = valid[tt] ? load16(Vc + row + (sub + 8 * cc) * 8) : u32x4{0, 0, 0, 0};
      }
    }

    // scores of the two tokens for every head of the group
    float s[GW][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float kf[NE];
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[cc * 8 + 2 * e] = T::lo(kx[tt][cc][e]);
          kf[cc * 8 + 2 * e + 1] = T::hi(kx[tt][cc][e]);
        }
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) a = fmaf(qf[g][e], kf[e], a);
        a = sum8(a);
        s[g][tt] = valid[tt] ? a * c : -__builtin_inff();
      }
    }

    // wave-uniform running max per head
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float mx = fmaxf(s[g][0], s[g][1]);
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (mx > m_run[g]) {
        const float alpha = fast_exp2(m_run[g] - mx);
        l_run[g] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[g][e] *= alpha;
        m_run[g] = mx;
      }
    }

    // weights and the weighted sum of values
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float vf[NE];
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[cc * 8 + 2 * e] = T::lo(vx[tt][cc][e]);
          vf[cc * 8 + 2 * e + 1] = T::hi(vx[tt][cc][e]);
        }
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float p = fast_exp2(s[g][tt] - m_run[g]);
        l_run[g] += p;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
      }
    }
  }

  // Sum over the 8 token slots (lanes with equal `sub`); m is wave-uniform.
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    float l = l_run[g];
    l += __shfl_xor(l, 8);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_run[g] = l;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float x = acc[g][e];
      x += __shfl_xor(x, 8);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[g][e] = x;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      if (sub == 0) {
        red_m[w][g] = m_run[g];
        red_l[w][g] = l_run[g];
      }
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) red_acc[w][g][(sub + 8 * cc) * 8 + e] = acc[g][cc * 8 + e];
    }
  }
  __syncthreads();

  // Merge the 4 waves' states; one thread per (head, column).
  for (int x = tid; x < GW * D; x += kDecThreads) {
    const int g = x / D, col = x % D;
    float M = red_m[0][g];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) M = fmaxf(M, red_m[ww][g]);
    float l = 0.f, a = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float f = fast_exp2(red_m[ww][g] - M);
      l = fmaf(f, red_l[ww][g], l);
      a = fmaf(f, red_acc[ww][g][col], a);
    }
    const size_t slot_idx = ((size_t)seq * Hq + h0 + g) * max_splits + split;
    part_acc[slot_idx * D + col] = a;
    if (col == 0) {
      part_m[slot_idx] = M;
      part_l[slot_idx] = l;
    }
  }
}

// One wave per (sequence, query head): merge the splits' (m, l, acc).
template <class T, int D>
__global__ __launch_bounds__(64) void fa_decode_merge(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_acc, const int32_t* __restrict__ seq_lens, int Hq,
    int split_tokens, int max_splits, uint16_t* __restrict__ O) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x, seq = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = seq_lens[seq];
  const int ns = min(max((L + split_tokens - 1) / split_tokens, 0), max_splits);
  const size_t base = ((size_t)seq * Hq + h) * max_splits;

  float M = kSentinel;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_m[base + s]);
  float l = 0.f, a[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) a[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float f = fast_exp2(part_m[base + s] - M);
    l = fmaf(f, part_l[base + s], l);
#pragma unroll
    for (int e = 0; e < PER; ++e) a[e] = fmaf(f, part_acc[(base + s) * D + lane * PER + e], a[e]);
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = O + ((size_t)seq * Hq + h) * D + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow) = T::pack(a[0] * inv, a[1] * inv);
  } else {
    const uint32_t x = T::pack(a[0] * inv, 0.f);
    orow[0] = (uint16_t)(x & 0xffffu);
  }
}

// ---------------------------------------------------------------------------
// plan and launchers
// ---------------------------------------------------------------------------
DecodePlan decode_plan(int num_seqs, int heads_q, int heads_kv, int max_blocks_per_seq,
                       int block_size) {
  DecodePlan p;
  const int group = heads_q / heads_kv;
  p.heads_per_wg = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  p.subgroups = group / p.heads_per_wg;
  const long long max_tokens = (long long)max_blocks_per_seq * block_size;
  // 512 keys per split; smaller when the batch alone cannot fill the GPU.
  int st = 512;
  const long long base = (long long)num_seqs * heads_kv * p.subgroups;
  while (st > 64 && base * ((max_tokens + st - 1) / st) < 2048) st /= 2;
  p.split_tokens = st;
  p.max_splits = (int)((max_tokens + st - 1) / st);
  return p;
}

size_t decode_workspace_bytes(const DecodePlan& p, int num_seqs, int heads_q, int dv) {
  return (size_t)num_seqs * heads_q * p.max_splits * (size_t)(dv + 2) * sizeof(float);
}

template <class T, int D, int GW>
static hipError_t launch_dec(const DecodeArgs& a, const DecodePlan& p) {
  float* part_m = (float*)a.workspace;
  float* part_l = part_m + (size_t)a.num_seqs * a.heads_q * p.max_splits;
  float* part_acc = part_l + (size_t)a.num_seqs * a.heads_q * p.max_splits;
  const float c = a.scale * kLog2e;
  dim3 grid1(p.max_splits, a.heads_kv * p.subgroups, a.num_seqs);
  hipLaunchKernelGGL((fa_decode_split<T, D, GW>), grid1, dim3(kDecThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.block_size,
                     a.heads_q, a.heads_kv, a.heads_q / a.heads_kv, p.subgroups,
                     a.max_blocks_per_seq, a.num_blocks, p.split_tokens, p.max_splits, c, part_m,
                     part_l, part_acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.heads_q, a.num_seqs);
  hipLaunchKernelGGL((fa_decode_merge<T, D>), grid2, dim3(64), 0, (hipStream_t)a.stream,
                     part_m, part_l, part_acc, a.seq_lens, a.heads_q, p.split_tokens,
                     p.max_splits, (uint16_t*)a.o);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t dispatch_gw(const DecodeArgs& a, const DecodePlan& p) {
  if (p.heads_per_wg == 4) return launch_dec<T, D, 4>(a, p);
  if (p.heads_per_wg == 2) return launch_dec<T, D, 2>(a, p);
  return launch_dec<T, D, 1>(a, p);
}

hipError_t launch_decode(const DecodeArgs& a) {
  const DecodePlan p =
      decode_plan(a.num_seqs, a.heads_q, a.heads_kv, a.max_blocks_per_seq, a.block_size);
  if (a.dtype == 2) return a.d == 128 ? dispatch_gw<BF16, 128>(a, p) : dispatch_gw<BF16, 64>(a, p);
  return a.d == 128 ? dispatch_gw<F16, 128>(a, p) : dispatch_gw<F16, 64>(a, p);
}

}  // namespace fa
