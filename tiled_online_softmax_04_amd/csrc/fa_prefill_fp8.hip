// FP8 prefill attention for gfx950 (CDNA4): Q, K, V stored as OCP E4M3 codes
// with one float32 descale factor per tensor; O in float32, float16 or
// bfloat16.  The pages name FP8 only as something FlashAttention-3 added on
// Hopper (llminference.xinbetween.com S12, production list); the computation
// is the same tiled single pass with the online-softmax update as the 16-bit
// kernel (10100.com section 7), on the real inputs descale * decode(code).
//
// Shape: one workgroup of 8 waves (two per SIMD) owns 256 query rows of one
// (batch, head); each wave keeps its 32 query rows in VGPRs for the whole key
// loop.  64-key K/V tiles stream through a four-stage LDS ring filled by
// buffer loads that write LDS directly: two tiles are computed between
// barriers while the next two land.
// Both products run on v_mfma_f32_32x32x64_f8f6f4 (64 fp8 products per lane
// per instruction, twice the bf16 rate):
//   S^T = K Q^T: per 32-key block, d/64 MFMAs; K rows come from LDS (32
//     bytes per lane, kappa row order), Q^T from registers;
//   O^T += V^T P^T: per 32-column block of O, one MFMA over all 64 keys; V^T
//     from transposing byte reads of LDS (ds_read_b64_tr_b8: each lane gets
//     one column of 8 consecutive keys), P rounded to E4M3 in registers.
// The running sum l adds the same rounded P through one more MFMA against an
// all-ones operand: it matches the P.V product term for term and costs one
// matrix instruction instead of unpacking 32 codes per lane on the VALU.
//
// Scales: the fp32 scores are exact sums of code products; c = scale *
// q_descale * k_descale * log2(e) turns them into log2-domain scores, and the
// epilogue multiplies by v_descale / l.  The running max is raised lazily
// (slack 8, as in the 16-bit kernel), so weights stay at most 2^8 = 256: inside
// the E4M3 range (finite up to 448; the conversion gives NaN only from 464
// up) and, for the key at the row max, an exact power of two.

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {

namespace {

constexpr int kW8 = 8;           // waves per workgroup
constexpr int kT8 = 64 * kW8;    // threads per workgroup
constexpr int kBr8 = 32 * kW8;   // query rows per workgroup
constexpr int kBc8 = 64;         // keys per tile
constexpr int kStages8 = 3;      // LDS ring depth
// Tiles computed between two barriers.  Two halve the barrier waits per
// tile; the ring then holds four stages, two computed while two land.
#ifndef FA8_GROUP
#define FA8_GROUP 2
#endif
constexpr int kGroup8 = FA8_GROUP;
constexpr int kRing8 = kGroup8 > 1 ? 2 * kGroup8 : kStages8;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(8 * sizeof(uint32_t)))) uint32_t u32x8;

template <int D>
struct Geo8 {
  static constexpr int kChunks = D / 16;                 // 16-byte chunks per row
  static constexpr int kTileBytes = kBc8 * D;            // one K (or V) tile
  static constexpr int kStageBytes = 2 * kTileBytes;     // K then V
  static constexpr int kRowsPerDma = 64 / kChunks;       // rows one wave-wide DMA covers
  static constexpr int kDmaPerTile = kBc8 / kRowsPerDma; // wave DMAs per K (or V) tile
  static constexpr int kDmaPerWave = 2 * kDmaPerTile / kW8;
  static_assert(kDmaPerWave >= 1 && 2 * kDmaPerTile % kW8 == 0 &&
                    kDmaPerTile % kDmaPerWave == 0,
                "each wave's DMAs must stay within the K or the V tile");
  static constexpr int kQSteps = D / 64;                 // MFMAs per 32-key block of S^T
  static constexpr int kOTiles = D / 32;                 // 32-row blocks of O^T
};

// XOR swizzles of the 16-byte chunks of a row (rows are D bytes: 128 or 64)
// so that operand reads of LDS hit distinct banks (64 banks, 256 bytes per
// cycle):
//  - K, 16-byte reads, 16 lanes per cycle: 16 rows at one logical chunk.
//    Rows of 128 B put two rows side by side in the bank width; XOR with
//    (row / 2) % 8 spreads the 16 rows over the 16 slots (rows of 64 B: four
//    rows side by side, XOR with (row / 4) % 4);
//  - V, transposing 8-byte reads, 32 lanes per cycle: 8 consecutive rows at
//    two adjacent logical chunks.  XOR with 2 * ((row / 2) % 4) (64 B rows:
//    2 * ((row / 4) % 2)) keeps the pair of chunks adjacent and sends the rows
//    that share a bank offset to different chunk pairs.
template <int D>
__device__ __forceinline__ int k_swz8(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int v_swz8(int row) {
  return D == 128 ? (((row >> 1) & 3) << 1) : (((row >> 2) & 1) << 1);
}

__device__ __forceinline__ f32x16 mfma_fp8(u32x8 a, u32x8 b, f32x16 c) {
  // Zero scale operands select the unscaled v_mfma_f32_32x32x64_f8f6f4; format
  // code 0 is E4M3 for both operands.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0,
                                                         0, 0, 0, 0);
}

// Four floats to four E4M3 codes (round to nearest even), first in the low byte.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ u32x8 cat(u32x4 a, u32x4 b) {
  return u32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace

// OUT: 0 float32, 1 float16, 2 bfloat16.
template <int D, bool CAUSAL, bool RAGGED, int OUT>
__global__ __launch_bounds__(kT8, 2) void fa_fwd_fp8(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    void* __restrict__ O, const int32_t* __restrict__ seq_lens, int Hq, int group, int n, int m,
    int q_tiles, int total, float c, float v_descale) {
  using G = Geo8<D>;
  __shared__ __align__(16) uint8_t smem[kRing8 * G::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, hf = lane >> 5;

  // Units (batch, query head, Q tile), Q tiles fastest; KV groups dealt to
  // the XCDs in turn.
  const int logical = CAUSAL ? xcd_heavy_first(blockIdx.x, total, group * q_tiles, q_tiles)
                             : xcd_by_group(blockIdx.x, total, group * q_tiles);
  const int bh = logical / q_tiles;
  const int qt_ord = logical % q_tiles;
  const int qt = CAUSAL ? q_tiles - 1 - qt_ord : qt_ord;  // longest causal rows first
  const int b = bh / Hq, h = bh % Hq;
  const int Hkv = Hq / group;
  const size_t q_base = ((size_t)b * Hq + h) * (size_t)n * D;
  const size_t kv_base = ((size_t)b * Hkv + h / group) * (size_t)m * D;

  const int pad =
      RAGGED ? __builtin_amdgcn_readfirstlane(min(max(n - seq_lens[b], 0), n)) : 0;
  const int wg_q0 = qt * kBr8;
  const int wg_q1 = min(n, wg_q0 + kBr8);
  const int wq0 = wg_q0 + w * 32;
  const int qrow = wq0 + ql;
  const bool q_ok = qrow < n && qrow >= pad;

  const int key_lo = pad;  // keys before the left pad are never attended
  const int key_hi = m;
  const int kv_end = CAUSAL ? min(key_hi, wg_q1) : key_hi;
  const bool no_keys = (RAGGED && wg_q1 <= pad) || kv_end <= key_lo;
  const int t_begin = key_lo / kBc8;
  const int t_end = no_keys ? t_begin : (kv_end + kBc8 - 1) / kBc8;

  // K and V of this head as buffers over exactly [key_lo, m): padding rows
  // and rows past the end read back as zeros.
  const uint32_t kv_bytes = (uint32_t)max(key_hi - key_lo, 0) * (uint32_t)D;

  // DMA of a tile into a ring stage: lane l fills LDS row p = first + l /
  // kChunks, physical chunk l % kChunks, with the key (kappa order for K) and
  // logical chunk that belong there.
  uint32_t dma_off[G::kDmaPerWave];
  const bool dma_v = w * G::kDmaPerWave >= G::kDmaPerTile;  // first half of the waves: K
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    const int ii = w * G::kDmaPerWave + i - (dma_v ? G::kDmaPerTile : 0);
    const int p = ii * G::kRowsPerDma + lane / G::kChunks;
    const int pc = lane % G::kChunks;
    const int key = dma_v ? p : ((p & ~31) | kappa(p & 31));
    const int chunk = pc ^ (dma_v ? v_swz8<D>(p) : k_swz8<D>(p));
    dma_off[i] = (uint32_t)(key * D + chunk * 16);
  }
  const u32x4 rsrc_dma_words = make_rsrc_words(
      (dma_v ? V : K) + kv_base + (size_t)key_lo * D, kv_bytes);
  lds_char* const lds = (lds_char*)smem;
  const int dma_lds0 = (dma_v ? G::kTileBytes : 0) +
                       (w * G::kDmaPerWave - (dma_v ? G::kDmaPerTile : 0)) * G::kRowsPerDma * D;
  auto issue_tile = [&](int t, int st) {
    const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds + st * G::kStageBytes + dma_lds0));
    // (t * kBc8 - key_lo) may be negative: it wraps past 2^31 and reads zeros.
    const uint32_t tile_off = (uint32_t)((t * kBc8 - key_lo) * D);
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i)
      dma16_untracked(rsrc_dma_words, tile_off + dma_off[i],
                      dst + (uint32_t)(i * G::kRowsPerDma * D));
  };
#pragma unroll
  for (int i = 0; i < (kGroup8 > 1 ? kGroup8 : kStages8 - 1); ++i)
    if (t_begin + i < t_end) issue_tile(t_begin + i, i);

  // Queries as B operands of S^T = K Q^T: lane holds query ql, 32 consecutive
  // d (bytes 64 ks + 32 hf ...) for each MFMA ks.
  u32x8 qT[G::kQSteps];
#pragma unroll
  for (int ks = 0; ks < G::kQSteps; ++ks) {
    const uint8_t* src = Q + q_base + (size_t)qrow * D + ks * 64 + hf * 32;
    qT[ks] = q_ok ? cat(load16(src), load16(src + 16)) : u32x8{};
  }

  f32x16 acc[G::kOTiles];
#pragma unroll
  for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2] = f32x16{};
  f32x16 lacc = f32x16{};  // every element: l of query ql
  float m_run = kSentinel; // running max, scaled log2 units
  const u32x8 ones = {0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u,
                      0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};  // E4M3 1.0

  // Per-lane LDS byte offsets of the operands within a stage.
  uint32_t k_off[G::kQSteps][2];  // K row ql, chunks 4 ks + 2 hf (+1)
#pragma unroll
  for (int ks = 0; ks < G::kQSteps; ++ks)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      k_off[ks][j] = (uint32_t)(ql * D + ((4 * ks + 2 * hf + j) ^ k_swz8<D>(ql)) * 16);
  uint32_t v_off[G::kOTiles];  // transposing V reads for keys 8 hf + 0..7
  {
    const int grp = lane >> 4, r = (lane & 15) >> 1, half = lane & 1;
    const int row = 8 * (grp >> 1) + r;
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2)
      v_off[t2] = (uint32_t)(row * D + (((2 * t2 + (grp & 1)) ^ v_swz8<D>(row)) * 16) + 8 * half);
  }

  wait_vm_lgkm0<0>();
  bare_barrier();

  // A whole wave above the causal diagonal, or wholly padding, skips a tile.
  auto wave_idle = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * kBc8;
    int all_pad = __builtin_amdgcn_readfirstlane(RAGGED && wq0 + 31 < pad);
    // Loop-invariant when not causal; evaluated in the loop all the same, so
    // that the compiler does not unswitch the loop on it (the second copy of
    // the loop body spills).
    asm volatile("" : "+s"(all_pad));
    return (CAUSAL && j0 > wq0 + 31) || all_pad != 0;
  };
  // S^T[key][query] of tile t (ring stage st) for 64 keys: two 32-key blocks.
  auto scores = [&](int st, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    const lds_char* Ks = lds + st * G::kStageBytes;
    sacc[0] = sacc[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < G::kQSteps; ++ks) {
      const u32x8 a0 = cat(*(const lds_u32x4*)(Ks + k_off[ks][0]),
                           *(const lds_u32x4*)(Ks + k_off[ks][1]));
      const u32x8 a1 = cat(*(const lds_u32x4*)(Ks + k_off[ks][0] + 32 * D),
                           *(const lds_u32x4*)(Ks + k_off[ks][1] + 32 * D));
      sacc[0] = mfma_fp8(a0, qT[ks], sacc[0]);
      sacc[1] = mfma_fp8(a1, qT[ks], sacc[1]);
    }
  };
  // The rest of tile t: mask, online softmax, P.V.
  auto finish = [&](int t, int st, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
    const int j0 = t * kBc8;
    {
      const lds_char* Vs = lds + st * G::kStageBytes + G::kTileBytes;

      // V^T operands: read g (0..3) covers keys 32 (g/2) + 16 (g%2) + 8 hf + 0..7.
      const uint32_t vs_addr = (uint32_t)(uintptr_t)Vs;
      u32x2 vr[4][G::kOTiles];
      auto issue_v = [&](auto Gc) __attribute__((always_inline)) {
        constexpr int g = decltype(Gc)::value;
        constexpr int off = (32 * (g >> 1) + 16 * (g & 1)) * D;
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) vr[g][t2] = lds_read_tr8(vs_addr + v_off[t2] + off);
      };
      __builtin_amdgcn_sched_barrier(0);
        static_for<0, 2>([&](auto Gc) __attribute__((always_inline)) { issue_v(Gc); });
        __builtin_amdgcn_sched_barrier(0);  // the V^T reads go out here

      // Mask only tiles that straddle the diagonal, the pad or the end of K.
      const bool need_mask = (CAUSAL && j0 + kBc8 - 1 > wq0) || (j0 + kBc8 > key_hi) ||
                             (j0 < key_lo);
      if (__builtin_expect(need_mask, 0)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = 16 * (i >> 3) + 8 * hf + (i & 7);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const int key = j0 + 32 * mt + kk;
            const bool bad = key >= key_hi || key < key_lo || (CAUSAL && key > qrow);
            sacc[mt][i] = bad ? -__builtin_inff() : sacc[mt][i];
          }
        }
      }

      // Online softmax: row max over this lane's 32 keys and the partner lane's.
      float a = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) a = fmaxf(a, fmaxf(sacc[0][i], sacc[0][i + 1]));
#pragma unroll
      for (int i = 0; i < 16; i += 2) a = fmaxf(a, fmaxf(sacc[1][i], sacc[1][i + 1]));
      const float mx = max_xor32(a) * c;
      if (__builtin_expect(__any(mx > m_run + kSlack), 0)) {
        asm volatile("" ::: "memory");  // a real branch, not a speculated rescale
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2] *= alpha;
        lacc *= alpha;
        m_run = m_new;
      }

      // P as E4M3 codes in the B-operand order: byte 8g + e is key
      // 32 (g/2) + 16 (g%2) + 8 hf + e, i.e. element 8 (g%2) + e of block g/2.
      u32x8 pb;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int i = 8 * (g & 1) + 4 * e2;
          pb[2 * g + e2] = pack_e4m3x4(fast_exp2(fmaf(sacc[g >> 1][i], c, -m_run)),
                                       fast_exp2(fmaf(sacc[g >> 1][i + 1], c, -m_run)),
                                       fast_exp2(fmaf(sacc[g >> 1][i + 2], c, -m_run)),
                                       fast_exp2(fmaf(sacc[g >> 1][i + 3], c, -m_run)));
        }
      }
      lacc = mfma_fp8(ones, pb, lacc);

      __builtin_amdgcn_sched_barrier(0);
        static_for<2, 4>([&](auto Gc) __attribute__((always_inline)) { issue_v(Gc); });
        __builtin_amdgcn_sched_barrier(0);  // the V^T reads go out here
      wait_lgkm0();
#pragma unroll
      for (int t2 = 0; t2 < G::kOTiles; ++t2) {
        const u32x8 va = {vr[0][t2][0], vr[0][t2][1], vr[1][t2][0], vr[1][t2][1],
                          vr[2][t2][0], vr[2][t2][1], vr[3][t2][0], vr[3][t2][1]};
        acc[t2] = mfma_fp8(va, pb, acc[t2]);
      }
    }
  };
  // One tile from ring stage st.
  auto tile = [&](int t, int st) __attribute__((always_inline)) {
    if (!wave_idle(t)) {
      f32x16 sacc[2];
      scores(st, sacc);
      finish(t, st, sacc);
    }
  };

#if FA8_GROUP > 1
  // kGroup8 tiles between barriers: they are computed from half of the ring
  // while the next kGroup8 land in the other half.
  for (int t = t_begin; t < t_end; t += kGroup8) {
    const int it = t - t_begin;
#pragma unroll
    for (int g = 0; g < kGroup8; ++g)
      if (t + kGroup8 + g < t_end) issue_tile(t + kGroup8 + g, (it + kGroup8 + g) % kRing8);
#pragma unroll
    for (int g = 0; g < kGroup8; ++g)
      if (t + g < t_end) tile(t + g, (it + g) % kRing8);
    wait_vm_lgkm0<0>();
    bare_barrier();
  }
#else
  for (int t = t_begin; t < t_end; ++t) {
    const int it = t - t_begin;
    const bool pre = t + kStages8 - 1 < t_end;
    if (pre) issue_tile(t + kStages8 - 1, (it + kStages8 - 1) % kStages8);
    tile(t, it % kStages8);
    // This wave's part of tile t+1 has landed and its reads of stage st are
    // done; after the barrier every wave may read t+1 and refill stage st.
    if (pre) {
      wait_vm_lgkm0<(kStages8 - 2) * G::kDmaPerWave>();
    } else {
      wait_vm_lgkm0<0>();
    }
    bare_barrier();
  }
#endif

  // -------- epilogue: O = acc * v_descale / l, zero for rows without keys --------
  if (qrow >= n) return;
  const float l = lacc[0];
  const float f = (l > 0.f && q_ok) ? v_descale / l : 0.f;
#pragma unroll
  for (int t2 = 0; t2 < G::kOTiles; ++t2) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv0 = 32 * t2 + 8 * g + 4 * hf;
      const size_t off = q_base + (size_t)qrow * D + dv0;
      const float x0 = acc[t2][4 * g] * f, x1 = acc[t2][4 * g + 1] * f;
      const float x2 = acc[t2][4 * g + 2] * f, x3 = acc[t2][4 * g + 3] * f;
      if constexpr (OUT == 0) {
        *reinterpret_cast<float4*>(static_cast<float*>(O) + off) = float4{x0, x1, x2, x3};
      } else if constexpr (OUT == 1) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(O) + off) =
            u32x2{F16::pack(x0, x1), F16::pack(x2, x3)};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(O) + off) =
            u32x2{BF16::pack(x0, x1), BF16::pack(x2, x3)};
      }
    }
  }
}

namespace {

template <int D, bool C, bool R, int OUT>
hipError_t launch_fp8(const Fp8Args& a) {
  const int q_tiles = (a.n + kBr8 - 1) / kBr8;
  const long long total = (long long)a.batch * a.heads_q * q_tiles;
  const double c = (double)a.scale * (double)a.q_descale * (double)a.k_descale *
                   1.4426950408889634;
  hipLaunchKernelGGL((fa_fwd_fp8<D, C, R, OUT>), dim3((unsigned)total), dim3(kT8), 0,
                     (hipStream_t)a.stream, (const uint8_t*)a.q, (const uint8_t*)a.k,
                     (const uint8_t*)a.v, a.o, a.seq_lens, a.heads_q, a.heads_q / a.heads_kv,
                     a.n, a.m, q_tiles, (int)total, (float)c, a.v_descale);
  return hipGetLastError();
}

template <int D, int OUT>
hipError_t dispatch_fp8_mask(const Fp8Args& a) {
  const bool r = a.seq_lens != nullptr;
  if (a.causal) return r ? launch_fp8<D, true, true, OUT>(a) : launch_fp8<D, true, false, OUT>(a);
  return r ? launch_fp8<D, false, true, OUT>(a) : launch_fp8<D, false, false, OUT>(a);
}

template <int D>
hipError_t dispatch_fp8_out(const Fp8Args& a) {
  if (a.out_dtype == 0) return dispatch_fp8_mask<D, 0>(a);
  if (a.out_dtype == 1) return dispatch_fp8_mask<D, 1>(a);
  return dispatch_fp8_mask<D, 2>(a);
}

}  // namespace

long long fwd_fp8_grid_size(int batch, int heads_q, int n) {
  return (long long)batch * heads_q * ((n + kBr8 - 1) / kBr8);
}

hipError_t launch_fwd_fp8(const Fp8Args& a) {
  return a.d == 128 ? dispatch_fp8_out<128>(a) : dispatch_fp8_out<64>(a);
}

}  // namespace fa
