// FP8 prefill attention for gfx950 (CDNA4): Q, K, V stored as OCP E4M3 codes
// with one float32 descale factor per tensor; O in float32, float16 or
// bfloat16.  The pages name FP8 only as something FlashAttention-3 added on
// Hopper (llminference.xinbetween.com S12, production list); the computation
// is the same tiled single pass with the online-softmax update as the 16-bit
// kernel (10100.com section 7), on the real inputs descale * decode(code).
//
// Shape: one workgroup of 8 waves (two per SIMD) owns 256 query rows of one
// (batch, head); each wave keeps its 32 query rows in VGPRs for the whole key
// loop.  64-key K/V tiles stream through an LDS ring filled by buffer loads
// that write LDS directly, two tiles (or pipeline steps) per barrier.  At
// d = 128 the key loop is a software pipeline, as in the 16-bit kernel: each
// step issues the next tile's score MFMAs beside this tile's exponentials and
// E4M3 packing, then this tile's P.V MFMAs beside the next tile's exp2
// arguments (five stages: the tiles of both steps and the one whose scores
// the second step forms, while the next two land).  At d = 64 a step
// would hold half as many MFMAs for the same vector work, and whole tiles are
// computed in turn from one half of a four-stage ring while the other lands.
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
// epilogue multiplies by v_descale / l.  The running max is raised lazily.
// The d = 64 loop raises it when a tile's max beats it by more than 8 (as in
// the 16-bit kernel), so weights stay at most 2^8 = 256.  The pipelined d = 128
// loop forms no tile max at all: it exponentiates against the running max as
// it stands and raises it only when a weight reached 464, the first value the
// E4M3 conversion turns into NaN (the format has no infinity; finite values
// end at 448), which the l product then carries.  Weights from 448 up to 464
// round to 448, within the format's 2^-4 relative rounding.

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {

namespace {

constexpr int kW8 = 8;           // waves per workgroup
constexpr int kT8 = 64 * kW8;    // threads per workgroup
constexpr int kBr8 = 32 * kW8;   // query rows per workgroup
constexpr int kBc8 = 64;         // keys per tile
constexpr int kGroup8 = 2;       // tiles (or pipeline steps) between two barriers
// d = 128 runs the software-pipelined key loop: at a barrier tiles t, t+1,
// t+2 are in the ring (the second step forms the scores of t+2) while t+3,
// t+4 land, five stages.  d = 64 computes two whole tiles between barriers
// from one half of a four-stage ring while the next two land.
template <int D>
constexpr bool pipelined8() {
  return D == 128;
}
template <int D>
constexpr int ring8() {
  return pipelined8<D>() ? 2 * kGroup8 + 1 : 2 * kGroup8;
}

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
  constexpr bool kPipe = pipelined8<D>();
  constexpr int kRing8 = ring8<D>();
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
  for (int i = 0; i < (kPipe ? kGroup8 + 1 : kGroup8); ++i)
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

  const float c_scale = c;
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

  if constexpr (!kPipe) {
    // kGroup8 tiles between barriers: they are computed from half of the
    // ring while the next kGroup8 land in the other half.
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
  } else {
    // Software pipeline over the key tiles, kGroup8 steps between barriers.
    // At a barrier tiles t .. t+kGroup8 are in the ring (the last step forms
    // the scores of tile t+kGroup8), and tiles t+kGroup8+1 .. t+2 kGroup8 go
    // into the stages that the steps before the barrier finished with.
    int t_wave_end = t_end;  // tiles this wave computes: [t_begin, t_wave_end)
    if (wq0 >= n) t_wave_end = t_begin;
    if constexpr (CAUSAL) t_wave_end = min(t_wave_end, (wq0 + 31) / kBc8 + 1);
    if constexpr (RAGGED)
      if (wq0 + 31 < pad) t_wave_end = t_begin;
    t_wave_end = __builtin_amdgcn_readfirstlane(max(t_wave_end, t_begin));
    auto ring = [](int x) __attribute__((always_inline)) { return x >= kRing8 ? x - kRing8 : x; };

    // Masked scores of a tile that straddles the diagonal, the pad or the
    // end of K become -inf.
    auto needs_mask = [&](int t) __attribute__((always_inline)) {
      const int j0 = t * kBc8;
      return (CAUSAL && j0 + kBc8 - 1 > wq0) || (j0 + kBc8 > key_hi) || (j0 < key_lo);
    };
    auto mask = [&](int t, f32x16 (&sc)[2]) __attribute__((always_inline)) {
      const int j0 = t * kBc8;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 16 * (i >> 3) + 8 * hf + (i & 7);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int key = j0 + 32 * mt + kk;
          const bool bad = key >= key_hi || key < key_lo || (CAUSAL && key > qrow);
          sc[mt][i] = bad ? -__builtin_inff() : sc[mt][i];
        }
      }
    };
    // Row max of one 32-key block: this lane's 16 scores in max3 steps.
    auto max16 = [](const f32x16& x) __attribute__((always_inline)) {
      float a = fmaxf(fmaxf(x[0], x[1]), x[2]);
      float b = fmaxf(fmaxf(x[3], x[4]), x[5]);
      float d = fmaxf(fmaxf(x[6], x[7]), x[8]);
      a = fmaxf(fmaxf(a, x[9]), x[10]);
      b = fmaxf(fmaxf(b, x[11]), x[12]);
      d = fmaxf(fmaxf(d, x[13]), x[14]);
      return fmaxf(fmaxf(fmaxf(a, b), d), x[15]);
    };

    // One step of the pipeline.  On entry sa holds tile t's exp2 arguments
    // s * c - m (formed in the step before, or the prologue).
    //  block A: tile t+1's S^T MFMAs beside tile t's weights exp2(arg) and
    //           their E4M3 packing, then tile t's l MFMA;
    //  the rare branch that raises the running max (see the file header);
    //  block C: tile t's P.V MFMAs beside tile t+1's exp2 arguments
    //           (written over sb).
    // Scheduling fences fix the order: after every MFMA, one slice of the
    // vector work.  The last tile of a wave still forms the scores of the
    // stage after it (never used), so that a step is straight-line code.
    constexpr int kSlotsA = 2 * G::kQSteps;  // MFMAs of block A
    constexpr int kSlotsC = G::kOTiles;      // MFMAs of block C
    static_assert(kSlotsA == 4 && kSlotsC == 4, "the step's slices assume d = 128");
    auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    auto step = [&](int t, int st_v, int st_k, f32x16 (&sa)[2], f32x16 (&sb)[2])
                    __attribute__((always_inline)) {
      const bool next = t + 1 < t_wave_end;
      // V^T operands of tile t: read g (0..3) covers keys 32 (g/2) + 16 (g%2)
      // + 8 hf + 0..7, the constant part of the address in the instruction.
      const lds_char* Vst = lds + st_v * G::kStageBytes + G::kTileBytes;
      u32x2 vr[4][G::kOTiles];
      auto vread = [&](int g) __attribute__((always_inline)) {
        const int off = (32 * (g >> 1) + 16 * (g & 1)) * D;
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2)
          vr[g][t2] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                                    (lds_i32x2*)(Vst + v_off[t2] + off)));
      };
      // K operands of tile t+1.
      const lds_char* Kst = lds + st_k * G::kStageBytes;
      u32x8 ka[G::kQSteps][2];
      auto kread = [&](int ks) __attribute__((always_inline)) {
        ka[ks][0] = cat(*(const lds_u32x4*)(Kst + k_off[ks][0]),
                        *(const lds_u32x4*)(Kst + k_off[ks][1]));
        ka[ks][1] = cat(*(const lds_u32x4*)(Kst + k_off[ks][0] + 32 * D),
                        *(const lds_u32x4*)(Kst + k_off[ks][1] + 32 * D));
      };

      // ---------------- block A ----------------
      // Word w of the E4M3 weights holds elements 4 (w % 4) .. +3 of score
      // block w / 4 (the B-operand order, see the packing in finish()).
      // Item c: the exponentials of word c (c < 8) and the packing of word
      // c - 1 (c >= 1).
      float pe[2][4];
      u32x8 pb;
      auto valu_a = [&](int cc) __attribute__((always_inline)) {
        if (cc < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[cc & 1][e] = fast_exp2(sa[cc >> 2][4 * (cc & 3) + e]);
        }
        if (cc >= 1) {
          const int wd = cc - 1, h2 = wd & 1;
          // The first conversion keeps the upper half of its destination,
          // which the second one overwrites: it may be any register, and
          // pe[h2][0]'s, which dies here, saves clearing one.
          const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(pe[h2][0], pe[h2][1],
                                                              __float_as_uint(pe[h2][0]), false);
          pb[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(pe[h2][2], pe[h2][3], lo, true);
        }
      };
      // Item 0 before the first MFMA, while its K operands are read; then
      // two items after each MFMA, the next k-step's K operands one step
      // ahead, and the V^T reads once the first K operands are consumed.
      kread(0);
      valu_a(0);
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" ::"v"(pe[0][e]));  // before the first MFMA
      fence();
#pragma unroll
      for (int slot = 0; slot < kSlotsA; ++slot) {
        const int ks = slot >> 1, hh = slot & 1;
        sb[hh] = mfma_fp8(ka[ks][hh], qT[ks], ks == 0 ? f32x16{} : sb[hh]);
        fence();
        valu_a(2 * slot + 1);
        valu_a(2 * slot + 2);
        if (hh == 0 && ks + 1 < G::kQSteps) kread(ks + 1);
        if (slot == 1) {
          vread(0);
          vread(1);
        }
        if (slot == 2) {
          vread(2);
          vread(3);
        }
        fence();
      }
      // The weights are formed here, beside the MFMAs: an empty use keeps
      // the compiler from sinking them below the branch that follows.
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) asm volatile("" ::"v"(pb[wd]));
      const float l_old = lacc[0];
      lacc = mfma_fp8(ones, pb, lacc);
      fence();

      if (__builtin_expect(next && needs_mask(t + 1), 0)) mask(t + 1, sb);

      // A weight that reached 464 converted to NaN (E4M3 has no infinity),
      // and the l product carried it: the tile beat the running max by more
      // than log2(464).  Rare: raise the max of the rows whose arguments pass
      // kSlack to their tile max, rescale, and form the weights again.
      const uint32_t lbits = __float_as_uint(lacc[0]) & 0x7fffffffu;
      if (__builtin_expect(__any(lbits > 0x7f800000u), 0)) {
        asm volatile("" ::: "memory");  // a real branch
        const float a_max = max_xor32(fmaxf(max16(sa[0]), max16(sa[1])));
        const float shift = a_max > kSlack ? a_max : 0.f;
        const float alpha = fast_exp2(-shift);
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2] *= alpha;
#pragma unroll
        for (int i = 0; i < 32; ++i) sa[i >> 4][i & 15] -= shift;
#pragma unroll
        for (int cc = 0; cc < 9; ++cc) valu_a(cc);
        const float l_new = l_old * alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) lacc[i] = l_new;
        lacc = mfma_fp8(ones, pb, lacc);
        m_run += shift;
      }

      // ---------------- block C ----------------
      // The exp2 arguments of tile t+1 against the running max, 8 after each
      // P.V MFMA.
#pragma unroll
      for (int slot = 0; slot < kSlotsC; ++slot) {
        const int t2 = slot;
        const u32x8 va = {vr[0][t2][0], vr[0][t2][1], vr[1][t2][0], vr[1][t2][1],
                          vr[2][t2][0], vr[2][t2][1], vr[3][t2][0], vr[3][t2][1]};
        acc[t2] = mfma_fp8(va, pb, acc[t2]);
#pragma unroll
        for (int i = 8 * slot; i < 8 * slot + 8; ++i)
          sb[i >> 4][i & 15] = fmaf(sb[i >> 4][i & 15], c_scale, -m_run);
        fence();
      }
      // The arguments are formed here, beside the MFMAs (see above).
#pragma unroll
      for (int i = 0; i < 32; ++i) asm volatile("" ::"v"(sb[i >> 4][i & 15]));
    };

    f32x16 sa[2], sb[2];
    // Prologue: tile t_begin's scores and arguments (acc and l are still
    // zero: nothing to rescale).
    if (t_begin < t_wave_end) {
      scores(0, sa);
      if (needs_mask(t_begin)) mask(t_begin, sa);
      const float mxc = max_xor32(fmaxf(max16(sa[0]), max16(sa[1]))) * c_scale;
      m_run = fmaxf(mxc, m_run);
#pragma unroll
      for (int i = 0; i < 32; ++i) sa[i >> 4][i & 15] = fmaf(sa[i >> 4][i & 15], c_scale, -m_run);
    }
    int s0 = 0;  // ring stage of tile t
    for (int t = t_begin; t < t_end; t += kGroup8) {
#pragma unroll
      for (int g = 1; g <= kGroup8; ++g)
        if (t + kGroup8 + g < t_end) issue_tile(t + kGroup8 + g, ring(s0 + kGroup8 + g));
#pragma unroll
      for (int g = 0; g < kGroup8; ++g) {
        if (t + g < t_wave_end) {
          // The two score buffers swap roles from step to step.
          if (g % 2 == 0) step(t + g, ring(s0 + g), ring(s0 + g + 1), sa, sb);
          else step(t + g, ring(s0 + g), ring(s0 + g + 1), sb, sa);
        }
      }
      static_assert(kGroup8 % 2 == 0, "the arguments are back in sa after a group");
      // This wave's DMAs are done and its LDS reads finished: after the
      // barrier tiles t+kGroup8 .. t+2 kGroup8 are readable and the stages
      // of tiles t .. t+kGroup8-1 free.
      wait_vm_lgkm0<0>();
      bare_barrier();
      s0 = ring(s0 + kGroup8);
    }
  }

  // -------- epilogue: O = acc * v_descale / l, zero for rows without keys --------
  const float l = lacc[0];
  const float f = (l > 0.f && q_ok) ? v_descale / l : 0.f;
  if constexpr (OUT == 0) {
    // float32 rows: twice the ring's room, so straight from the accumulators
    if (qrow >= n) return;
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const size_t off = q_base + (size_t)qrow * D + 32 * t2 + 8 * g + 4 * hf;
        *reinterpret_cast<float4*>(static_cast<float*>(O) + off) =
            float4{acc[t2][4 * g] * f, acc[t2][4 * g + 1] * f, acc[t2][4 * g + 2] * f,
                   acc[t2][4 * g + 3] * f};
      }
    }
  } else {
    // 16-bit rows leave through the idle ring, whole rows per store (RowStage).
    using RS = RowStage<D * 2>;
    static_assert(kW8 * RS::kBytes <= kRing8 * G::kStageBytes, "staged O fits the ring");
    using T = typename std::conditional<OUT == 1, F16, BF16>::type;
    wait_vm_lgkm0<0>();
    bare_barrier();  // every wave is done with the ring
    lds_char* const ob = lds + w * RS::kBytes;
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // columns 32 t2 + 8 g + 4 hf .. +3 of row ql
        const uint32_t lo = T::pack(acc[t2][4 * g] * f, acc[t2][4 * g + 1] * f);
        const uint32_t hi = T::pack(acc[t2][4 * g + 2] * f, acc[t2][4 * g + 3] * f);
        RS::put(ob, ql, (32 * t2 + 8 * g + 4 * hf) * 2, u32x2{lo, hi});
      }
    }
    RS::store(ob, lane,
              reinterpret_cast<char*>(static_cast<uint16_t*>(O) + q_base + (size_t)wq0 * D),
              (size_t)D * 2, n - wq0);
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
