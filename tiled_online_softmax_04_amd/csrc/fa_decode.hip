// Paged grouped-query decode for gfx950: split-K partial pass + merge pass.
//
// One query token per sequence.  The keys of a sequence live in a paged cache
// reached through its block table (the S12 chapter's paged loop, "实现"); the
// query heads of one group share a KV head and read each K/V row once
// ("它如何与你已经搭好的部分组合").  Decode has a single query row, so the
// parallelism comes from the keys instead (flash-decoding, S12): the key range
// of a sequence is cut into splits, each split runs the online-softmax
// recurrence in its own workgroup and leaves a partial state (m, l, o = acc / l),
// and a second kernel merges the partials with the same rescale (S12
// exercise 1).
//
// This pass moves about 4 FLOP per byte, far below the MFMA ridge point, so it
// is bandwidth bound: the kernel streams K/V with 16-byte loads straight into
// VGPRs and does the arithmetic on the vector ALUs.
//
// Lane layout of the split kernel: a wave takes 16 consecutive tokens at a
// time.  Each lane owns one 16-byte column chunk of a row (kLpt = d/8 lanes
// cover a 256- or 128-byte row) for kTpl tokens of the chunk: lane =
// kLpt * slot + sub handles tokens slot, slot + kSlots, ... and chunk sub, so
// one load instruction reads kSlots whole rows.
//  - q.k: v_dot2 on packed 16-bit pairs, finished by a DPP sum over the kLpt
//    lanes of a token;
//  - p.v: the tokens of a lane are paired, so one v_dot2 adds
//    p(t0) v(t0) + p(t1) v(t1) for one column (p rounded to the input type,
//    as the prefill's P.V MFMA does, and l sums the same rounded values);
//  - the running max is wave-uniform and raised only when some score beats it
//    by more than kSlack (a wave vote), so the common path has no cross-lane
//    max at all;
//  - a wave loads a chunk and then uses it, with no software prefetch: that
//    keeps the kernel near 100 VGPRs, so four waves share each SIMD and keep
//    enough loads in flight (measured 1.4% faster than holding two chunks in
//    registers at three waves per SIMD).  The split's block-table entries
//    are staged in LDS once;
//  - K/V rows are read once per call, so their loads are marked nontemporal:
//    the stream then does not push the partial states, written while it runs,
//    out of the caches (measured: 10% faster than plain loads);
//  - a split's partial state is stored as fp32 m, l and o = acc / l, so the
//    output is rounded to the 16-bit type once, in the merge.  (Rounding o to
//    16 bits here as well would add a second rounding of the same size as the
//    final one: for outputs in [2, 4) in bf16 the two together can exceed
//    1e-2.)

#include <mutex>

#include "../../include/fa.h"
#include "fa_common.h"
#include "fa_launch.h"

// The workspace of fa_paged_decode_noalloc: the split states in a static
// device array.  Every GPU the library runs on holds its own copy from the
// moment the code object is loaded there until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only stands in
// for the symbol); it passes the device address decode_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace fa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};  // per device; null until looked up
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

constexpr int kDecWaves = 8;  // per split: 8 chunks of 16 tokens each in flight
constexpr int kDecThreads = 64 * kDecWaves;
#ifndef FA_DECODE_CHUNK
#define FA_DECODE_CHUNK 16
#endif
constexpr int kDecChunk = FA_DECODE_CHUNK;  // tokens per wave step
#ifndef FA_DECODE_SPLIT
#define FA_DECODE_SPLIT 768
#endif
#ifndef FA_DECODE_WAVES_PER_EU
#define FA_DECODE_WAVES_PER_EU 4
#endif
// Keys per split: this, or a halving of it when the batch is small.  768 (six
// 16-token chunks per wave) measured 2% faster than 512, and 4% faster than
// 1024, on 64 sequences of 512-8192 keys (32 query heads, 8 KV heads, d = 128):
// fewer workgroups end on their split-state stores, and the last round of
// workgroups is still short.
constexpr int kMaxSplitTokens = FA_DECODE_SPLIT;
constexpr int kMaxSplitBlocks = kMaxSplitTokens + 1;

// 16-byte load of data used once per call (the K/V stream): nontemporal.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D>
struct DecGeo {
  static constexpr int kLpt = D / 8;              // lanes per token row
  static constexpr int kSlots = 64 / kLpt;        // token slots per wave
  static constexpr int kTpl = kDecChunk / kSlots; // tokens per lane per chunk
  static_assert(kTpl % 2 == 0, "tokens of a lane are paired");
};

template <int LPT>
__device__ __forceinline__ float sum_row(float x) {
  if constexpr (LPT == 16) return sum16(x);
  else return sum8(x);
}
// Sum / max over the token slots of a wave (lanes that share `sub`).
template <int LPT>
__device__ __forceinline__ float sum_slots(float x) {
  if constexpr (LPT == 8) x = sum_xor8(x);
  return sum_xor32(sum_xor16(x));
}
template <int LPT>
__device__ __forceinline__ float max_slots(float x) {
  if constexpr (LPT == 8) x = max_xor8(x);
  return max_xor32(max_xor16(x));
}

// POW2: block_size is 1 << bs_shift, so block and slot indices are a shift
// and a mask rather than an integer division per token.
template <class T, int D, int GW, bool POW2>
__global__ __launch_bounds__(kDecThreads, FA_DECODE_WAVES_PER_EU) void fa_decode_split(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int bs, int bs_shift, int Hq, int Hkv, int group, int subgroups,
    int maxb, int num_blocks, int split_tokens, int max_splits, float c,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ part_o) {
  using G = DecGeo<D>;
  constexpr int TPL = G::kTpl;
  __shared__ int bt_s[kMaxSplitBlocks];
  __shared__ float red_m[kDecWaves][GW];
  __shared__ float red_l[kDecWaves][GW];
  __shared__ float red_acc[kDecWaves][GW][D];

  // KV heads (and head subgroups) vary fastest across workgroup ids, so the
  // workgroups reading the rows of one cache block run side by side.
  const int split = blockIdx.y;
  const int kvh = blockIdx.x / subgroups;
  const int sg = blockIdx.x % subgroups;
  const int seq = blockIdx.z;
  const int L = seq_lens[seq];
  const int tok0 = split * split_tokens;
  if (tok0 >= L) return;  // empty split: the merge never reads it
  const int tok1 = min(L, tok0 + split_tokens);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = lane / G::kLpt, sub = lane % G::kLpt;
  const int h0 = kvh * group + sg * GW;  // first query head of this workgroup

  // Physical blocks of this split.  Entries and lengths outside their stated
  // ranges are clamped so that no access leaves the buffers.
  const int blk0 = POW2 ? tok0 >> bs_shift : tok0 / bs;
  const int nblk = (POW2 ? (tok1 - 1) >> bs_shift : (tok1 - 1) / bs) - blk0 + 1;
  const int32_t* bt = block_table + (size_t)seq * maxb;
  for (int i = tid; i < nblk; i += kDecThreads)
    bt_s[i] = min(max(bt[min(blk0 + i, maxb - 1)], 0), num_blocks - 1);

  // Query values at this lane's 8 dims, packed 16-bit pairs.
  u32x4 qp[GW];
#pragma unroll
  for (int g = 0; g < GW; ++g) qp[g] = load16(Q + ((size_t)seq * Hq + h0 + g) * D + sub * 8);

  float m_run[GW], l_run[GW], acc[GW][8];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m_run[g] = kSentinel;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  const size_t row_stride = (size_t)Hkv * D;
  // K/V chunks of this lane's tokens in the 16-token chunk at t0, block ids
  // from the table staged in LDS.  Tokens past tok1 read a valid row (tok0)
  // and are masked out of the softmax.
  auto load_chunk = [&](int t0, u32x4 (&kx)[TPL], u32x4 (&vx)[TPL]) {
#pragma unroll
    for (int tt = 0; tt < TPL; ++tt) {
      int tok = t0 + slot + G::kSlots * tt;
      tok = tok < tok1 ? tok : tok0;
      const int blk = POW2 ? tok >> bs_shift : tok / bs;
      const int in_blk = tok - blk * bs;
      const int phys = bt_s[blk - blk0];
      // Row index of the token in the cache: fits 32 bits for any cache that
      // fits in device memory.
      const uint32_t row = (uint32_t)phys * (uint32_t)bs + (uint32_t)in_blk;
      const size_t off = (size_t)row * row_stride + (size_t)(kvh * D + sub * 8);
      kx[tt] = load16_stream(Kc + off);
      vx[tt] = load16_stream(Vc + off);
    }
  };

  // One chunk: scores, the lazy max, weights and the weighted sum of values.
  auto consume = [&](int t0, const u32x4 (&kx)[TPL], const u32x4 (&vx)[TPL]) {
    // scores of this lane's tokens for every head of the group
    float s[GW][TPL];
    bool raise = false;
#pragma unroll
    for (int tt = 0; tt < TPL; ++tt) {
      const bool valid = t0 + slot + G::kSlots * tt < tok1;
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        float a0 = T::dot2(qp[g][0], kx[tt][0], 0.f);
        float a1 = T::dot2(qp[g][1], kx[tt][1], 0.f);
        a0 = T::dot2(qp[g][2], kx[tt][2], a0);
        a1 = T::dot2(qp[g][3], kx[tt][3], a1);
        const float a = sum_row<G::kLpt>(a0 + a1);
        s[g][tt] = valid ? a * c : -__builtin_inff();
        raise = raise || s[g][tt] > m_run[g] + kSlack;
      }
    }
    // Rare: raise the wave-uniform running max to the chunk max.
    if (__builtin_expect(__any(raise), 0)) {
      asm volatile("" ::: "memory");  // a real branch, not a speculated rescale
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        float mx = s[g][0];
#pragma unroll
        for (int tt = 1; tt < TPL; ++tt) mx = fmaxf(mx, s[g][tt]);
        mx = max_slots<G::kLpt>(mx);
        const float m_new = fmaxf(m_run[g], mx);
        const float alpha = fast_exp2(m_run[g] - m_new);
        l_run[g] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
        m_run[g] = m_new;
      }
    }
    // weights of token pairs, packed, and the paired weighted sum of values
#pragma unroll
    for (int pr = 0; pr < TPL / 2; ++pr) {
      uint32_t pp[GW];
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        pp[g] = T::pack(fast_exp2(s[g][2 * pr] - m_run[g]), fast_exp2(s[g][2 * pr + 1] - m_run[g]));
        l_run[g] = T::add_pair(pp[g], l_run[g]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a = vx[2 * pr][e], b = vx[2 * pr + 1][e];
        const uint32_t lo = (a & 0xffffu) | (b << 16);      // column 2e of both tokens
        const uint32_t hi = (a >> 16) | (b & 0xffff0000u);  // column 2e+1
#pragma unroll
        for (int g = 0; g < GW; ++g) {
          acc[g][2 * e] = T::dot2(pp[g], lo, acc[g][2 * e]);
          acc[g][2 * e + 1] = T::dot2(pp[g], hi, acc[g][2 * e + 1]);
        }
      }
    }
  };

  // The waves take the 16-token chunks of the split in turn.
  constexpr int kStep = kDecWaves * kDecChunk;
  __syncthreads();  // block-table entries staged in LDS
  for (int t0 = tok0 + w * kDecChunk; t0 < tok1; t0 += kStep) {
    u32x4 kx[TPL], vx[TPL];
    load_chunk(t0, kx, vx);
    consume(t0, kx, vx);
  }

  // Sum over the token slots (lanes sharing `sub`); m is wave-uniform.
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    l_run[g] = sum_slots<G::kLpt>(l_run[g]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = sum_slots<G::kLpt>(acc[g][e]);
  }
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      if (sub == 0) {
        red_m[w][g] = m_run[g];
        red_l[w][g] = l_run[g];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red_acc[w][g][sub * 8 + e] = acc[g][e];
    }
  }
  __syncthreads();

  // Merge the waves' states; one thread per (head, column).  The split's
  // output o = acc / l goes out in fp32; l >= 1 for a split that holds keys
  // (its largest key has weight exp2(0) = 1).
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
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t slot_idx = ((size_t)seq * Hq + h0 + g) * max_splits + split;
    part_o[slot_idx * D + col] = a * inv;
    if (col == 0) {
      part_m[slot_idx] = M;
      part_l[slot_idx] = l;
    }
  }
}

constexpr int kMergeFast = 16;  // splits the merge reads in one go

// One wave per (sequence, query head): merge the splits' (m, l, o).  Lane s
// reads split s's (m, l); the weights 2^(m_s - M) l_s are shared across the
// wave and every lane sums its D/64 columns of the o_s over the splits, eight
// splits' loads in flight at a time: O = sum w_s l_s o_s / sum w_s l_s.
template <class T, int D>
__global__ __launch_bounds__(64) void fa_decode_merge(
    const float* __restrict__ part_m, const float* __restrict__ part_l,
    const float* __restrict__ part_o, const int32_t* __restrict__ seq_lens, int Hq,
    int split_tokens, int max_splits, uint16_t* __restrict__ O) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x, seq = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = seq_lens[seq];
  const int ns = min(max((L + split_tokens - 1) / split_tokens, 0), max_splits);
  const size_t base = ((size_t)seq * Hq + h) * max_splits;

  uint16_t* orow = O + ((size_t)seq * Hq + h) * D + lane * PER;
  // This lane's PER fp32 columns of one split's o.
  auto load_o = [&](const float* row, float (&x)[PER]) {
    if constexpr (PER == 2) {
      const f32x2 pr = *reinterpret_cast<const f32x2*>(row + lane * PER);
      x[0] = pr[0];
      x[1] = pr[1];
    } else {
      x[0] = row[lane];
    }
  };
  auto store = [&](const float (&a)[PER], float inv) {
    if constexpr (PER == 2) {
      *reinterpret_cast<uint32_t*>(orow) = T::pack(a[0] * inv, a[1] * inv);
    } else {
      const uint32_t x = T::pack(a[0] * inv, 0.f);
      orow[0] = (uint16_t)(x & 0xffffu);
    }
  };
  if (ns <= kMergeFast) {
    // Up to kMergeFast splits (every sequence of up to 12288 keys at 768-key
    // splits): all loads go out at once -- (m, l) of split `lane` and this
    // lane's columns of every split's o -- so the pass waits out one memory
    // latency instead of three.  Splits at or past ns re-read split ns - 1
    // (in bounds, written by this call) and weigh 0.
    float a[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) a[e] = 0.f;
    if (ns == 0) {  // no keys: O = 0
      store(a, 0.f);
      return;
    }
    const bool mine = lane < ns;
    const float ms = mine ? part_m[base + lane] : -__builtin_inff();
    const float lsv = mine ? part_l[base + lane] : 0.f;
    float x[kMergeFast][PER];
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) load_o(part_o + (base + min(u, ns - 1)) * D, x[u]);
    float M = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float wgt = mine ? fast_exp2(ms - M) * lsv : 0.f;
    float l = wgt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) {
      const float wu = __shfl(wgt, u);
#pragma unroll
      for (int e = 0; e < PER; ++e) a[e] = fmaf(wu, x[u][e], a[e]);
    }
    store(a, l > 0.f ? 1.f / l : 0.f);
    return;
  }

  // pass 1: the largest running max over all splits
  float M = -__builtin_inff();
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, part_m[base + s]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  // pass 2: weights 2^(m_s - M) l_s, 64 splits at a time (one per lane)
  float a[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) a[e] = 0.f;
  float l = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const float wgt = s < ns ? fast_exp2(part_m[base + s] - M) * part_l[base + s] : 0.f;
    l += wgt;
    const int cnt = min(64, ns - s0);
    for (int j0 = 0; j0 < cnt; j0 += 8) {
      float x[8][PER], wj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // Past cnt: re-read the last split (in bounds, written by this call)
        // and give it weight 0.
        const int j = min(j0 + u, cnt - 1);
        wj[u] = j0 + u < cnt ? __shfl(wgt, j0 + u) : 0.f;
        load_o(part_o + (base + s0 + j) * D, x[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) a[e] = fmaf(wj[u], x[u][e], a[e]);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
  store(a, l > 0.f ? 1.f / l : 0.f);
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
  // kMaxSplitTokens keys per split; smaller when the batch alone cannot fill
  // the GPU with 2048 workgroups.
  int st = kMaxSplitTokens;
  const long long base = (long long)num_seqs * heads_kv * p.subgroups;
  while (st > 64 && base * ((max_tokens + st - 1) / st) < 2048) st /= 2;
  p.split_tokens = st;
  p.max_splits = (int)((max_tokens + st - 1) / st);
  return p;
}

size_t decode_workspace_bytes(const DecodePlan& p, int num_seqs, int heads_q, int dv) {
  // part_m, part_l and part_o, all fp32
  return (size_t)num_seqs * heads_q * p.max_splits * (2 + (size_t)dv) * sizeof(float);
}

template <class T, int D, int GW>
static hipError_t launch_dec(const DecodeArgs& a, const DecodePlan& p) {
  const int bs = a.block_size;
  const bool pow2 = (bs & (bs - 1)) == 0;
  const int shift = pow2 ? __builtin_ctz((unsigned)bs) : -1;
  float* part_m = (float*)a.workspace;
  float* part_l = part_m + (size_t)a.num_seqs * a.heads_q * p.max_splits;
  float* part_o = part_l + (size_t)a.num_seqs * a.heads_q * p.max_splits;
  const float c = a.scale * kLog2e;
  dim3 grid1(a.heads_kv * p.subgroups, p.max_splits, a.num_seqs);
  auto kernel = pow2 ? &fa_decode_split<T, D, GW, true> : &fa_decode_split<T, D, GW, false>;
  hipLaunchKernelGGL(kernel, grid1, dim3(kDecThreads), 0,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, bs, shift,
                     a.heads_q, a.heads_kv, a.heads_q / a.heads_kv, p.subgroups,
                     a.max_blocks_per_seq, a.num_blocks, p.split_tokens, p.max_splits, c, part_m,
                     part_l, part_o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid2(a.heads_q, a.num_seqs);
  hipLaunchKernelGGL((fa_decode_merge<T, D>), grid2, dim3(64), 0, (hipStream_t)a.stream,
                     part_m, part_l, part_o, a.seq_lens, a.heads_q, p.split_tokens,
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
