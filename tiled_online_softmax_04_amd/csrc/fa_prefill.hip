// Prefill attention kernels for gfx950 (CDNA4).
//
// fa_fwd_mfma: bf16 / fp16 inputs.  One workgroup of 8 waves (two per SIMD)
// owns 256 query rows of one (batch, head); each wave owns 32 of them and
// keeps them resident in VGPRs as MFMA operands ("Q 常驻片上寄存器", 10100.com
// section 7).  64-key K/V tiles stream through a ring of LDS stages: each
// wave moves its share of a tile with buffer loads that write LDS directly (no
// VGPR round trip).  Per tile the wave forms S^T = K Q^T with
// v_mfma_f32_32x32x16, applies the online-softmax update of the same section
// (running max, rescale of the history by exp(m_old - m_new), running sum) and
// accumulates O^T += V^T P^T with a second MFMA whose V^T operands come from
// transposing LDS reads.  The key loop is a software pipeline over the tiles
// (one barrier per tile, four stages): tile t+1's scores are formed beside
// tile t's exponentials, and tile t's P.V beside tile t+1's row max.  This
// holds for contiguous K/V and for paged K/V whose block table fits in LDS
// after the ring; a larger table takes a loop of one tile per barrier over
// three stages, two tiles ahead, with the softmax between the two products.
// Tiles wholly above the causal diagonal or wholly inside a left pad are never
// visited (10100.com section 6).
//
// Why S^T rather than S: in the 32x32 MFMA accumulator each lane holds one
// column and 16 rows.  With keys as rows and queries as columns every lane
// holds 16 keys of ONE query, so the row max and row sum of the softmax are
// lane-local plus one exchange with the lane 32 away, and the probabilities
// come out already in the layout the P.V MFMA wants as its B operand (after a
// fixed permutation of the K rows in LDS, see kappa()).
//
// fa_fwd_f32: float32 inputs, for which fp32 scores are not accurate enough on
// "hot" data (scores of several hundred).  Scores, the running max and the
// shifted exponent are float64; so are the weights and the accumulator.

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {

// ---------------------------------------------------------------------------
// MFMA kernel geometry
// ---------------------------------------------------------------------------
#ifndef FA_PREFILL_WAVES
#define FA_PREFILL_WAVES 8
#endif
#ifndef FA_PREFILL_QPW
#define FA_PREFILL_QPW 32
#endif
constexpr int kWaves = FA_PREFILL_WAVES;    // waves per workgroup
constexpr int kQPerWave = FA_PREFILL_QPW;   // queries per wave (32-column MFMA tiles)
constexpr int kNT = kQPerWave / 32;         // query tiles per wave
constexpr int kBr = kQPerWave * kWaves;     // query rows per workgroup
constexpr int kBc = 64;                     // keys per tile
constexpr int kThreads = 64 * kWaves;
#ifndef FA_PREFILL_STAGES
#define FA_PREFILL_STAGES 3
#endif
// LDS ring of K/V tiles: tile t is computed while tiles t+1 .. t+kStages-1 land.
constexpr int kStages = FA_PREFILL_STAGES;
static_assert(kStages == 2 || kStages == 3, "ring depth");
// LDS stages of the K/V ring: four for the software pipeline (contiguous K/V,
// and paged K/V whose block table fits beside the ring), three for the paged
// form with a large block table (one tile per barrier, two tiles ahead).
constexpr int ring_stages(bool tile_loop) { return tile_loop ? kStages : 4; }

template <int D>
struct Geo {
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kTileElems = kBc * D;             // one K (or V) tile
  static constexpr int kStageElems = 2 * kTileElems;     // K then V
  static constexpr int kRowsPerDma = 64 / kChunks;       // rows one wave-wide DMA covers
  static constexpr int kDmaPerTile = kBc / kRowsPerDma;  // wave DMAs per K (or V) tile
  static constexpr int kDmaPerWave = 2 * kDmaPerTile / kWaves;
  static_assert(2 * kDmaPerTile % kWaves == 0 && kDmaPerTile % kDmaPerWave == 0,
                "each wave's DMAs must stay within the K or the V tile");
  static constexpr int kQSteps = D / 16;                 // k-steps of S^T = K Q^T
  static constexpr int kOTiles = D / 32;                 // 32-row tiles of O^T
};

// XOR swizzles of the 16-byte chunks of a row, so that the MFMA operand reads
// hit distinct banks of the 64-bank (256 bytes per cycle) LDS:
//  - K: a 16-byte read serves 16 lanes per cycle, 16 rows at one logical
//    chunk; rows are 256 B (d = 128: 16 chunks) or 128 B (d = 64: two rows
//    share the bank width), so the XOR spreads 16 rows over 16 slots;
//  - V: a transposing read serves 32 lanes per cycle, 4 rows x 4 chunks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// The b-th longest of a batch's B sequences (lengths clamped to [0, cap], ties
// by index), for batches of up to 64: the workgroups of the longest
// sequences are handed out first, so that the short ones fill the end of the
// launch.  Larger batches keep their order.  Wave-uniform.
__device__ __forceinline__ int kth_longest(int b, const int32_t* __restrict__ lens, int B,
                                           int cap) {
  if (B > 64) return b;
  const int lane = threadIdx.x & 63;
  const int mine = lane < B ? min(max(lens[lane], 0), cap) : -1;
  int rank = 0;
  for (int i = 0; i < B; ++i) {
    const int li = __builtin_amdgcn_readlane(mine, i);
    rank += (li > mine || (li == mine && i < lane)) ? 1 : 0;
  }
  const unsigned long long hit = __ballot(lane < B && rank == b);
  return hit ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit)) : b;
}

// PARTIAL: attend only to keys in [key_begin, key_end) and write the result
// normalised over that range as float32 (Of) together with the natural-log
// softmax denominator of the range (Lse), instead of the final O.
// PG (paged): 0 for contiguous K and V.  Otherwise K and V are paged caches
// [num_blocks, bs, Hkv, D] reached through block_table; the n query rows of
// sequence b are its last n tokens (row i is token seq_lens[b] - n + i) and
// the causal mask is aligned to that.  PG = 1 runs the software-pipelined key
// loop (block table of up to kMaxPipelinedPagedBlocks entries, staged in LDS
// beside the four-stage ring), PG = 2 the one-tile-per-barrier loop over a
// three-stage ring for tables of up to kMaxPagedBlocks entries.
template <class T, int D, bool CAUSAL, bool RAGGED, bool PARTIAL, int PG>
#ifndef FA_PREFILL_WAVES_PER_EU
#define FA_PREFILL_WAVES_PER_EU (kWaves / 4)
#endif
__global__ __launch_bounds__(kThreads, FA_PREFILL_WAVES_PER_EU) void fa_fwd_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ Of,
    float* __restrict__ Lse, const int32_t* __restrict__ seq_lens, int Hq, int group, int n,
    int m, int key_begin, int key_end, int q_tiles, int total, float c,
    const int32_t* __restrict__ block_table, int bs, int bs_shift, int maxb, int num_blocks) {
  using G = Geo<D>;
  constexpr bool PAGED = PG != 0;
  constexpr int kRing = ring_stages(PG == 2);
  extern __shared__ __align__(16) uint16_t smem[];

  // Persistent form (dense, non-causal, full output): a launch of fewer
  // workgroups than units, each taking units blockIdx.x, + gridDim.x, ...  A
  // unit's output rows wait in registers and are stored after the next unit's
  // query and first tile copies have gone out, so the stores overlap its start.
  constexpr bool kPersist = !CAUSAL && !RAGGED && !PARTIAL && PG == 0;
  using RS16 = RowStage<D * 2>;
  u32x4 o_pend[RS16::kReads];
  __amdgpu_buffer_rsrc_t o_pend_rsrc;
  bool have_pend = false;

  for (int unit = blockIdx.x; unit < total; unit += gridDim.x) {
  int tid_ = threadIdx.x;
  // Per unit, so that nothing lane-derived is kept live across units (which
  // made the compiler spill).
  if constexpr (kPersist) asm volatile("" : "+v"(tid_));
  const int tid = tid_;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int ql = lane & 31, hf = lane >> 5;

  // Work units are (batch, query head, Q tile), Q tiles fastest; the units of
  // one KV group (batch, KV head) are consecutive.
  const int logical = CAUSAL ? xcd_heavy_first(unit, total, group * q_tiles, q_tiles)
                             : xcd_by_group(unit, total, group * q_tiles);
  const int bh = logical / q_tiles;
  const int qt_ord = logical % q_tiles;
  // Causal tiles further down hold more keys: hand those out first.
  const int qt = CAUSAL ? q_tiles - 1 - qt_ord : qt_ord;
  const int h = bh % Hq;
  // Sequences of different lengths: the longest first (see kth_longest).
  const int b = (RAGGED || PAGED)
                    ? kth_longest(bh / Hq, seq_lens, total / (Hq * q_tiles), RAGGED ? n : maxb * bs)
                    : bh / Hq;
  const int hkv = h / group;
  const int Hkv = Hq / group;

  const size_t q_base = ((size_t)b * Hq + h) * (size_t)n * D;
  const size_t kv_base = PAGED ? 0 : ((size_t)b * Hkv + hkv) * (size_t)m * D;
  const uint16_t* Qh = Q + q_base;
  const uint16_t* Kh = K + kv_base;
  const uint16_t* Vh = V + kv_base;

  // Padding rows of a left-padded sequence; out-of-range lengths are clamped.
  const int pad =
      RAGGED ? __builtin_amdgcn_readfirstlane(min(max(n - seq_lens[b], 0), n)) : 0;
  // Paged chunk: key position of query row i is qoff + i, qoff = L - n.
  const int L = PAGED ? __builtin_amdgcn_readfirstlane(min(max(seq_lens[b], 0), maxb * bs)) : 0;
  const int qoff = PAGED ? L - n : 0;
  const int wg_q0 = qt * kBr;
  const int wg_q1 = min(n, wg_q0 + kBr);
  const int wq0 = wg_q0 + w * kQPerWave;  // first query of this wave
  int qrow[kNT];
  bool q_ok[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    qrow[nt] = wq0 + 32 * nt + ql;
    // Rows that hold no real query: past n, inside the left pad, or (paged)
    // before the first token of the sequence.
    q_ok[nt] = qrow[nt] < n && (PAGED ? qrow[nt] + qoff >= 0 : qrow[nt] >= pad);
  }

  // Keys this call may attend: [key_lo, key_hi) -- past the left pad and
  // inside the requested range (the whole of [0, m) for a full call).
  const int key_lo = PAGED ? 0 : max(RAGGED ? pad : 0, key_begin);
  const int key_hi = PAGED ? L : min(m, key_end);
  // Key range of this workgroup, in whole tiles.
  const int kv_begin = (key_lo / kBc) * kBc;
  const int kv_end = CAUSAL ? min(key_hi, wg_q1 + qoff) : key_hi;
  const bool no_keys = (RAGGED && wg_q1 <= pad) || (PAGED && wg_q1 + qoff <= 0) ||
                       kv_end <= key_lo;
  const int t_begin = kv_begin / kBc;
  const int t_end = no_keys ? t_begin : (kv_end + kBc - 1) / kBc;

  // K and V of this head as buffers over exactly [key_lo, key_hi): rows
  // before it (padding, or keys below the range) and from key_hi on read
  // back as zeros, so no tile ever needs clamping and padding contents never
  // reach the arithmetic.
  const uint32_t kv_bytes = (uint32_t)max(key_hi - key_lo, 0) * (uint32_t)(D * 2);

  // DMA of a tile into a ring stage.  Lane l of a wave DMA fills LDS row
  // p = first + l / kChunks, physical chunk l % kChunks, and fetches the key
  // and logical chunk that belong there (kappa rows for K, swizzled chunks for
  // both).  The per-lane byte offsets within a tile never change.
  uint32_t dma_off[G::kDmaPerWave];
  int dma_key[G::kDmaPerWave], dma_col[G::kDmaPerWave];  // paged: key in tile, first column
  const bool dma_v = w * G::kDmaPerWave >= G::kDmaPerTile;  // first half of the waves: K
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    const int ii = w * G::kDmaPerWave + i - (dma_v ? G::kDmaPerTile : 0);
    const int p = ii * G::kRowsPerDma + lane / G::kChunks;
    const int pc = lane % G::kChunks;
    const int klocal = dma_v ? p : ((p & ~31) | kappa(p & 31));
    const int chunk = pc ^ (dma_v ? v_swz<D>(p) : k_swz<D>(p));
    dma_off[i] = (uint32_t)(klocal * D + chunk * 8) * 2u;
    dma_key[i] = klocal;
    dma_col[i] = chunk * 8;
  }
  const u32x4 rsrc_dma_words =
      make_rsrc_words(dma_v ? Vh + (size_t)key_lo * D : Kh + (size_t)key_lo * D, kv_bytes);
  lds_char* const lds = (lds_char*)smem;
  const int dma_lds0 = (dma_v ? G::kTileElems : 0) * 2 +
                       (w * G::kDmaPerWave - (dma_v ? G::kDmaPerTile : 0)) *
                           G::kRowsPerDma * D * 2;
  // Paged: the sequence's block-table entries the tiles touch, staged in LDS
  // after the ring (clamped into [0, num_blocks)).
  typedef __attribute__((address_space(3))) int lds_int;
  lds_int* const bt_s = (lds_int*)(lds + kRing * G::kStageElems * 2);
  if constexpr (PAGED) {
    const int nblk = no_keys ? 0 : min((kv_end + bs - 1) / bs, maxb);
    for (int i = tid; i < nblk; i += kThreads)
      bt_s[i] = min(max(block_table[(size_t)b * maxb + i], 0), num_blocks - 1);
    __syncthreads();
  }
  const uint16_t* const cache_dma = dma_v ? V : K;
  // Paged, block size a power of two that divides the 64-key tile: a lane's
  // row keeps its offset inside its block from tile to tile, and its block is
  // table entry t * (64 / bs) + (key >> log2 bs).  The byte offset of the row
  // inside the block (head and columns included) is fixed per lane.
  const bool pg_fast = PAGED && bs_shift >= 0 && bs <= kBc;
  uint32_t pg_off[G::kDmaPerWave];
  const uint64_t pg_blk_bytes = (uint64_t)bs * (uint64_t)Hkv * D * 2;
  if constexpr (PAGED) {
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i)
      pg_off[i] = pg_fast ? (uint32_t)((((uint32_t)(dma_key[i] & (bs - 1)) * (uint32_t)Hkv +
                                         (uint32_t)hkv) * D + (uint32_t)dma_col[i]) * 2u)
                          : 0u;
  }
  auto issue_tile = [&](int t, int st) {
    lds_char* dst = lds + st * G::kStageElems * 2 + dma_lds0;
    if constexpr (PAGED) {
      if (pg_fast && (t + 1) * kBc <= kv_end) {
        // Every row of the tile is a key this workgroup needs: the table
        // entries first, one wait, then the copies.
        const int e0 = t << (6 - bs_shift);
        uint32_t ent[G::kDmaPerWave];
#pragma unroll
        for (int i = 0; i < G::kDmaPerWave; ++i) ent[i] = (uint32_t)bt_s[e0 + (dma_key[i] >> bs_shift)];
#pragma unroll
        for (int i = 0; i < G::kDmaPerWave; ++i) {
          const uint64_t a = (uint64_t)(uintptr_t)cache_dma + (uint64_t)ent[i] * pg_blk_bytes + pg_off[i];
          gdma16_untracked((const void*)(uintptr_t)a,
                           (uint32_t)__builtin_amdgcn_readfirstlane(
                               (uint32_t)(uintptr_t)(dst + i * G::kRowsPerDma * D * 2)));
        }
        return;
      }
      // Each row through the table; rows past the keys this workgroup needs
      // repeat its last key (masked later) so no address leaves the cache.
#pragma unroll
      for (int i = 0; i < G::kDmaPerWave; ++i) {
        int tok = t * kBc + dma_key[i];
        tok = tok < kv_end ? tok : kv_end - 1;
        const int blk = bs_shift >= 0 ? tok >> bs_shift : tok / bs;
        const size_t row = (size_t)bt_s[blk] * (size_t)bs + (size_t)(tok - blk * bs);
        gdma16_untracked(cache_dma + (row * Hkv + hkv) * D + dma_col[i],
                         (uint32_t)__builtin_amdgcn_readfirstlane(
                             (uint32_t)(uintptr_t)(dst + i * G::kRowsPerDma * D * 2)));
      }
    } else {
      const uint32_t tile_off = (uint32_t)((t * kBc - key_lo) * D * 2);
      const uint32_t lds0 =
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
#pragma unroll
      for (int i = 0; i < G::kDmaPerWave; ++i)
        dma16_untracked(rsrc_dma_words, tile_off + dma_off[i],
                        lds0 + (uint32_t)(i * G::kRowsPerDma * D * 2));
    }
  };

  if constexpr (PG == 2) {
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
      if (t_begin + i < t_end) issue_tile(t_begin + i, i);
  }

  // Queries as B operands of S^T = K Q^T: lane holds column ql, 8 consecutive
  // d.  The pipelined loop brings them in through LDS (below); the other loop
  // loads them straight into registers.
  u32x4 qT[kNT][G::kQSteps];
  if constexpr (PG == 2) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int ks = 0; ks < G::kQSteps; ++ks)
        qT[nt][ks] = q_ok[nt] ? load16(Qh + (size_t)qrow[nt] * D + ks * 16 + hf * 8)
                              : u32x4{0, 0, 0, 0};
  }

  f32x16 acc[G::kOTiles][kNT];
  float m_run[kNT], l_run[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2][nt] = f32x16{};
    m_run[nt] = kSentinel;  // running max (scaled log2 units)
    l_run[nt] = 0.f;        // this lane's half of the running sum
  }

  // Per-lane LDS byte offsets of the MFMA operands within a stage.
  uint32_t k_off[G::kQSteps];  // K rows ql (and +32) for each k-step
#pragma unroll
  for (int ks = 0; ks < G::kQSteps; ++ks)
    k_off[ks] = (uint32_t)(ql * D + (((2 * ks + hf) ^ k_swz<D>(ql)) * 8)) * 2u;
  uint32_t v_off[G::kOTiles];  // transposing V reads, k-step 0, first half
  {
    const int g = lane >> 4, i = lane & 15;
    const int key = 8 * (g >> 1) + (i >> 2);
    const int chunk = 2 * (g & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2)
      v_off[t2] = (uint32_t)(key * D + (((4 * t2 + chunk) ^ v_swz<D>(key)) * 8) + (i & 1) * 4) * 2u;
  }

  if constexpr (PG == 2) {
    wait_vm_lgkm0<0>();
    bare_barrier();

    // One tile from ring stage st: scores, online softmax, P.V.
    auto tile = [&](int t, int st) __attribute__((always_inline)) {
      const int j0 = t * kBc;
      // Whole wave above the causal diagonal, or wholly padding: nothing to add.
      const bool wave_idle = (CAUSAL && j0 > wq0 + qoff + kQPerWave - 1) ||
                             (RAGGED && wq0 + kQPerWave - 1 < pad) ||
                             (PAGED && wq0 + qoff + kQPerWave - 1 < 0);
      if (!wave_idle) {
        const lds_char* Ks = lds + st * G::kStageElems * 2;
        const lds_char* Vs = Ks + G::kTileElems * 2;

        // S^T[key][query]: 64 keys (two 32-row tiles) x kQPerWave queries.
        f32x16 sacc[2][kNT];
  #pragma unroll
        for (int nt = 0; nt < kNT; ++nt) sacc[0][nt] = sacc[1][nt] = f32x16{};
        // K operands in batches of four k-steps: a batch's LDS reads are all
        // issued before its MFMAs, so the MFMAs do not wait out one read's
        // latency each (left to itself the compiler pairs every read with the
        // MFMA that uses it).
        constexpr int KB = G::kQSteps < 4 ? G::kQSteps : 4;
        static_assert(G::kQSteps % KB == 0, "batch");
  #pragma unroll
        for (int kb = 0; kb < G::kQSteps; kb += KB) {
          u32x4 ka[KB][2];
  #pragma unroll
          for (int u = 0; u < KB; ++u) {
            ka[u][0] = *(const lds_u32x4*)(Ks + k_off[kb + u]);
            ka[u][1] = *(const lds_u32x4*)(Ks + k_off[kb + u] + 32 * D * 2);
          }
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int u = 0; u < KB; ++u)
  #pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
              sacc[0][nt] = T::mfma32x32x16(ka[u][0], qT[nt][kb + u], sacc[0][nt]);
              sacc[1][nt] = T::mfma32x32x16(ka[u][1], qT[nt][kb + u], sacc[1][nt]);
            }
        }

        // V^T operands through transposing reads: 2 reads per (k-step j, dv tile).
        const uint32_t vs_addr = (uint32_t)(uintptr_t)Vs;
        uint32_t va[G::kOTiles];
  #pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) va[t2] = vs_addr + v_off[t2];
        u32x2 vr[4][G::kOTiles][2];
        auto issue_v = [&](auto J) {
          constexpr int j = decltype(J)::value;
  #pragma unroll
          for (int t2 = 0; t2 < G::kOTiles; ++t2) {
            vr[j][t2][0] = lds_read_tr16(va[t2] + (16 * j) * D * 2);
            vr[j][t2][1] = lds_read_tr16(va[t2] + (16 * j + 4) * D * 2);
          }
        };
        auto mma_v = [&](auto J, const u32x4 (&pbr)[kNT][4]) {
          constexpr int j = decltype(J)::value;
  #pragma unroll
          for (int t2 = 0; t2 < G::kOTiles; ++t2) {
            const u32x4 a = {vr[j][t2][0][0], vr[j][t2][0][1], vr[j][t2][1][0], vr[j][t2][1][1]};
  #pragma unroll
            for (int nt = 0; nt < kNT; ++nt) acc[t2][nt] = T::mfma32x32x16(a, pbr[nt][j], acc[t2][nt]);
          }
        };
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, 2>([&](auto J) { issue_v(J); });
        __builtin_amdgcn_sched_barrier(0);  // the V^T reads go out here

        // Mask only tiles that straddle the diagonal, the pad or the end of K
        // (a real branch: most tiles need no mask at all).
        const bool need_mask = (CAUSAL && j0 + kBc - 1 > wq0 + qoff) || (j0 + kBc > key_hi) ||
                               (j0 < key_lo);
        if (__builtin_expect(need_mask, 0)) {
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 16 * (i >> 3) + 8 * hf + (i & 7);
  #pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
              const int key = j0 + 32 * mt + kk;
              const bool kbad = key >= key_hi || key < key_lo;
  #pragma unroll
              for (int nt = 0; nt < kNT; ++nt) {
                const bool bad = kbad || (CAUSAL && key > qrow[nt] + qoff);
                sacc[mt][nt][i] = bad ? -__builtin_inff() : sacc[mt][nt][i];
              }
            }
          }
        }

        // Online softmax: tile row max (lane-local + the partner lane 32 away).
        float mx[kNT];
        bool raise = false;
  #pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          float a = fmaxf(sacc[0][nt][0], sacc[0][nt][1]);
  #pragma unroll
          for (int i = 2; i < 16; i += 2) a = fmaxf(a, fmaxf(sacc[0][nt][i], sacc[0][nt][i + 1]));
  #pragma unroll
          for (int i = 0; i < 16; i += 2) a = fmaxf(a, fmaxf(sacc[1][nt][i], sacc[1][nt][i + 1]));
          mx[nt] = max_xor32(a) * c;
          raise = raise || mx[nt] > m_run[nt] + kSlack;
        }
        // Raise the running max only when the tile beats it by more than kSlack
        // (wave-uniform branch).  Weights are then at most 2^kSlack, and acc and
        // l always share the same m, so O = acc / l is unchanged.
        if (__builtin_expect(__any(raise), 0)) {
          // A real branch: without the barrier the compiler executes the
          // rescale on every tile with alpha = 1.
          asm volatile("" ::: "memory");
  #pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            const float m_new = fmaxf(m_run[nt], mx[nt]);
            const float alpha = fast_exp2(m_run[nt] - m_new);
            l_run[nt] *= alpha;
  #pragma unroll
            for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2][nt] *= alpha;
            m_run[nt] = m_new;
          }
        }

        // p = exp2(S*c - m) as the B operand of O^T += V^T P^T.  The running
        // sum adds the same rounded weights the MFMA uses (two per v_dot2).
        u32x4 pb[kNT][4];
  #pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          float ps0 = 0.f, ps1 = 0.f;
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 8 * (j & 1) + 2 * e;
              const float p0 = fast_exp2(fmaf(sacc[j >> 1][nt][i], c, -m_run[nt]));
              const float p1 = fast_exp2(fmaf(sacc[j >> 1][nt][i + 1], c, -m_run[nt]));
              pb[nt][j][e] = T::pack(p0, p1);
              if (e & 1) ps1 = T::add_pair(pb[nt][j][e], ps1);
              else ps0 = T::add_pair(pb[nt][j][e], ps0);  // two chains for latency
            }
          }
          l_run[nt] += ps0 + ps1;
        }

        // O^T += V^T P^T.  k-steps 0, 1 of V^T were requested before the
        // softmax; 2, 3 go out now and land during the first half of the MFMAs.
        __builtin_amdgcn_sched_barrier(0);
        static_for<2, 4>([&](auto J) { issue_v(J); });
        __builtin_amdgcn_sched_barrier(0);  // the V^T reads go out here
        wait_lgkm0();
        static_for<0, 2>([&](auto J) { mma_v(J, pb); });
        wait_lgkm0();
        static_for<2, 4>([&](auto J) { mma_v(J, pb); });
      }
    };
    for (int t = t_begin; t < t_end; ++t) {
      const int it = t - t_begin;
      // Refill the stage read in the previous iteration with tile t+kStages-1.
      const bool pre = t + kStages - 1 < t_end;
      if (pre) issue_tile(t + kStages - 1, (it + kStages - 1) % kStages);
      tile(t, it % kStages);
      // This wave's part of tile t+1 has landed and its reads of stage st are
      // done; after the barrier every wave may read t+1 and refill stage st.
      if (kStages == 3 && pre) {
        wait_vm_lgkm0<(kStages - 2) * G::kDmaPerWave>();  // tile t+2 may stay in flight
      } else {
        wait_vm_lgkm0<0>();
      }
      bare_barrier();
    }
  } else {
    // ---------------------------------------------------------------------
    // Contiguous K/V, or paged K/V with a small block table: a software
    // pipeline over key tiles, one barrier per tile, four LDS stages (tiles t
    // and t+1 in use, t+2 landing, t+3 being issued).  Each step issues the S^T MFMAs of tile t+1 beside tile t's
    // exponentials, packing and row sums, then tile t's P.V MFMAs beside
    // tile t+1's row max, running-max update and exp2 arguments, so that a
    // wave's vector work sits between its own MFMAs (measured on gfx950: a
    // few ordinary VALU instructions between two MFMAs of one wave cost no
    // MFMA time; exponentials cost about half their issue time).
    // ---------------------------------------------------------------------
    static_assert(kNT == 1, "the pipelined loop takes 32 queries per wave");
    constexpr int kRingP = 4;
    static_assert(kRing == kRingP, "LDS ring of the pipelined loop");
    // Tiles this wave computes: [t_begin, t_wave_end).  Later tiles lie wholly
    // above its causal diagonal; a wave of padding rows or rows past n
    // computes none.  It still moves its share of every tile and meets every
    // barrier.
    int t_wave_end = t_end;
    if (wq0 >= n) t_wave_end = t_begin;
    if constexpr (CAUSAL) t_wave_end = min(t_wave_end, (wq0 + qoff + kQPerWave - 1) / kBc + 1);
    if constexpr (RAGGED)
      if (wq0 + kQPerWave - 1 < pad) t_wave_end = t_begin;
    if constexpr (PAGED)  // rows before the sequence's first token
      if (wq0 + qoff + kQPerWave - 1 < 0) t_wave_end = t_begin;
    t_wave_end = __builtin_amdgcn_readfirstlane(max(t_wave_end, t_begin));

    // The wave's 32 query rows come in whole rows per DMA (a load straight
    // into the B-operand layout would touch 32 rows per instruction) into its
    // own part of ring stages 2 and 3, chunks swizzled as in a K tile, and
    // are read back with the K-operand offsets.  Rows before the first real
    // query (left pad, or before a paged sequence's first token) and rows
    // from n on lie outside the buffer and read as zeros.
    {
      static_assert(kWaves * 32 * D * 2 <= 2 * G::kStageElems * 2, "queries fit stages 2 and 3");
      constexpr int kQDma = 32 * D * 2 / 1024;
      const int qpad = RAGGED ? pad : PAGED ? min(max(-qoff, 0), n) : 0;
      const u32x4 rsrc_q =
          make_rsrc_words(Qh + (size_t)qpad * D, (uint32_t)(n - qpad) * (uint32_t)(D * 2));
      const uint32_t qs_addr = (uint32_t)__builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds + 2 * G::kStageElems * 2 + w * (32 * D * 2)));
#pragma unroll
      for (int i = 0; i < kQDma; ++i) {
        const int p = i * G::kRowsPerDma + lane / G::kChunks;
        const int chunk = (lane % G::kChunks) ^ k_swz<D>(p);
        // rows before qpad give a negative offset, which wraps out of range
        dma16_untracked(rsrc_q, (uint32_t)(((wq0 - qpad + p) * D + chunk * 8) * 2),
                        qs_addr + (uint32_t)(i * 1024));
      }
    }
    // Tiles t_begin and t_begin+1 follow; t_begin+2 goes to stage 2 once
    // every wave has read its queries (after the barrier below).
    const int pre = min(2, t_end - t_begin);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (t_begin + i < t_end) issue_tile(t_begin + i, i);
    // The previous unit's output rows (persistent form) go out behind them:
    // always RS16::kReads store instructions, so the counts below are exact.
    int stores = 0;
    if constexpr (kPersist) {
      if (have_pend) {
        RS16::store_buf(o_pend, lane, o_pend_rsrc);
        stores = RS16::kReads;
        have_pend = false;
      }
    }
    // Loads complete in issue order: the queries first.
    wait_vm_lgkm0_rt(pre * G::kDmaPerWave + stores);
    asm volatile("" ::: "memory");
    {
      const lds_char* const qs = lds + 2 * G::kStageElems * 2 + w * (32 * D * 2);
#pragma unroll
      for (int ks = 0; ks < G::kQSteps; ++ks) qT[0][ks] = *(const lds_u32x4*)(qs + k_off[ks]);
    }
    // Then tile t_begin; tile t_begin+1 and the stores may stay in flight.
    wait_vm_lgkm0_rt((pre == 2 ? G::kDmaPerWave : 0) + stores);
    bare_barrier();
    if (t_begin + 2 < t_end) issue_tile(t_begin + 2, 2);

    // LDS byte offsets of the MFMA operands from one register each.  The K
    // chunk of lane ql at k-step ks is (2 ks + hf) XOR the row's swizzle, so
    // its offset is k_off[0] ^ (ks << 5); the transposing V read of column
    // tile t2 sits at v_off[0] ^ (t2 << 6).  The XORed bits lie below the row
    // bits (rows of 128 or 256 bytes) and above the lane's own chunk bits,
    // and stage bases are multiples of 8 KB, so base + off ^ x = (base + off) ^ x.
    static_assert(D == 128 || D == 64, "head dims");
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    // S^T[key][query] of tile t from its ring stage: 64 keys (two 32-row
    // tiles) x 32 queries (the first tile, before the pipeline starts).
    auto scores = [&](int t, f32x16 (&sc)[2]) __attribute__((always_inline)) {
      const uint32_t kb =
          lds_base + ((t - t_begin) & (kRingP - 1)) * G::kStageElems * 2 + k_off[0];
      sc[0] = sc[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < G::kQSteps; ++ks) {
        const uint32_t ka_addr = kb ^ (uint32_t)(ks << 5);
        const u32x4 a0 = *(const lds_u32x4*)(uintptr_t)ka_addr;
        const u32x4 a1 = *(const lds_u32x4*)(uintptr_t)(ka_addr + 32 * D * 2);
        sc[0] = T::mfma32x32x16(a0, qT[0][ks], sc[0]);
        sc[1] = T::mfma32x32x16(a1, qT[0][ks], sc[1]);
      }
    };

    // Masked scores of a tile that straddles the diagonal, the pad or the
    // ends of the key range become -inf.
    auto mask = [&](int t, f32x16 (&sc)[2]) __attribute__((always_inline)) {
      const int j0 = t * kBc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 16 * (i >> 3) + 8 * hf + (i & 7);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int key = j0 + 32 * mt + kk;
          const bool bad = key >= key_hi || key < key_lo || (CAUSAL && key > qrow[0] + qoff);
          sc[mt][i] = bad ? -__builtin_inff() : sc[mt][i];
        }
      }
    };

    // Row max of a tile's scores, the running-max update, and the exp2
    // arguments s * c - m written over the scores.  The running max moves
    // only when the tile beats it by more than kSlack, so weights stay below
    // 2^kSlack; acc and l always share m, so O = acc / l does not depend on
    // where m sits.  Returns whether some row of the wave moved its max
    // (then acc and l must be rescaled by exp2(m_old - m_new)).
    const float c_scale = c;
    auto softmax_args = [&](f32x16 (&sc)[2], bool live, float& m_new)
                            __attribute__((always_inline)) {
      float a = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) a = fmaxf(a, fmaxf(sc[0][i], sc[0][i + 1]));
#pragma unroll
      for (int i = 0; i < 16; i += 2) a = fmaxf(a, fmaxf(sc[1][i], sc[1][i + 1]));
      const float mxc = max_xor32(a) * c;
      const bool raise = live && mxc > m_run[0] + kSlack;
      m_new = raise ? mxc : m_run[0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[mt][i] = fmaf(sc[mt][i], c, -m_new);
      return raise;
    };
    auto rescale = [&](float m_new) __attribute__((always_inline)) {
      const float alpha = fast_exp2(m_run[0] - m_new);  // 1 for rows that kept m
      l_run[0] *= alpha;
#pragma unroll
      for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2][0] *= alpha;
    };

    // One step of the pipeline.  On entry sa holds tile t's exp2 arguments
    // (formed in the step before, or the prologue).
    //  block A: tile t+1's S^T MFMAs beside tile t's weights p = exp2(arg),
    //           rounded to the input type as the B operand of the P.V MFMA,
    //           and their row sums (l adds the same rounded weights);
    //  block C: tile t's P.V MFMAs beside tile t+1's row max and arguments;
    //  then the rare rescale branch.
    // The instruction order inside each block is fixed by scheduling fences:
    // after every MFMA comes one slice of the vector work, and the LDS
    // operand reads run four (K) or two (V) k-steps ahead of their MFMAs, so
    // that the two waves of a SIMD keep the matrix core fed.  The last tile
    // of a wave still forms the scores of the stage after it (stale LDS,
    // never used): one surplus S^T product per wave and Q tile buys a
    // straight-line step.
    constexpr int kSlotsA = 2 * G::kQSteps;   // MFMAs of block A (16 or 8)
    constexpr int kSlotsC = 4 * G::kOTiles;   // MFMAs of block C (16 or 8)
    constexpr int kKpf = G::kQSteps < 4 ? G::kQSteps : 4;  // K k-steps ahead
    auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    auto step = [&](int t, f32x16 (&sa)[2], f32x16 (&sb)[2]) __attribute__((always_inline)) {
      const bool next = t + 1 < t_wave_end;

      // V^T operands of block C (tile t's stage); the first k-step's reads
      // go out at the end of block A.
      const uint32_t vb = lds_base + ((t - t_begin) & (kRingP - 1)) * G::kStageElems * 2 +
                          G::kTileElems * 2 + v_off[0];
      uint32_t vt[G::kOTiles];
#pragma unroll
      for (int t2 = 0; t2 < G::kOTiles; ++t2) vt[t2] = vb ^ (uint32_t)(t2 << 6);
      u32x4 va[4][G::kOTiles];
      auto vread = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) {
          const uint32_t a = vt[t2] + (16 * j) * D * 2;
          const u32x2 a0 = lds_read_tr16(a), a1 = lds_read_tr16(a + 4 * D * 2);
          va[j][t2] = u32x4{a0[0], a0[1], a1[0], a1[1]};
        }
      };

      // ---------------- block A ----------------
      const uint32_t kb = lds_base + ((t + 1 - t_begin) & (kRingP - 1)) * G::kStageElems * 2 +
                          k_off[0];
      u32x4 ka[G::kQSteps][2];
      auto kread = [&](int ks) __attribute__((always_inline)) {
        const uint32_t addr = kb ^ (uint32_t)(ks << 5);
        ka[ks][0] = *(const lds_u32x4*)(uintptr_t)addr;
        ka[ks][1] = *(const lds_u32x4*)(uintptr_t)(addr + 32 * D * 2);
      };
      float pe[32];
      u32x4 pb[4];
      float ps0 = 0.f, ps1 = 0.f;
      // Vector work of block A in 16 slices: exponentials (slices 0-7),
      // packs one slice behind them (2, 4, 6, 8), row sums (9-12).
      auto valu_a = [&](int c) __attribute__((always_inline)) {
        if (c < 8) {
          const int j = c >> 1, h = c & 1;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pe[8 * j + 4 * h + e] = fast_exp2(sa[j >> 1][8 * (j & 1) + 4 * h + e]);
        }
        if (c >= 2 && c <= 8 && (c & 1) == 0) {
          const int j = c / 2 - 1;
#pragma unroll
          for (int e = 0; e < 4; ++e) pb[j][e] = T::pack(pe[8 * j + 2 * e], pe[8 * j + 2 * e + 1]);
        }
        if (c >= 9 && c <= 12) {
          const int j = c - 9;
          ps0 = T::add_pair(pb[j][0], ps0);
          ps1 = T::add_pair(pb[j][1], ps1);
          ps0 = T::add_pair(pb[j][2], ps0);
          ps1 = T::add_pair(pb[j][3], ps1);
        }
        if (c == 13) l_run[0] += ps0 + ps1;
      };
#pragma unroll
      for (int ks = 0; ks < kKpf; ++ks) kread(ks);
      sb[0] = sb[1] = f32x16{};
      fence();
#pragma unroll
      for (int ks = 0; ks < G::kQSteps; ++ks) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int slot = 2 * ks + hh;
          sb[hh] = T::mfma32x32x16(ka[ks][hh], qT[0][ks], sb[hh]);
          if constexpr (kSlotsA == 16) {
            valu_a(slot);
          } else {
            valu_a(2 * slot);
            valu_a(2 * slot + 1);
          }
          if (hh == 1 && ks + kKpf < G::kQSteps) kread(ks + kKpf);
          fence();
        }
      }
      // The weights and l are formed here, beside the MFMAs: an empty use keeps
      // the compiler from sinking them below the branch that follows.
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(pb[j]));
      asm volatile("" ::"v"(l_run[0]));
      vread(0);
      fence();

      // Masked scores of tile t+1 (straddling the diagonal, the pad or the
      // ends of the key range) become -inf: a rare branch.
      const int j1 = (t + 1) * kBc;
      const bool need_mask = next && ((CAUSAL && j1 + kBc - 1 > wq0 + qoff) ||
                                      (j1 + kBc > key_hi) || (j1 < key_lo));
      if (__builtin_expect(need_mask, 0)) mask(t + 1, sb);

      // ---------------- block C ----------------
      // Vector work of block C in 16 slices: the row max of tile t+1 over its
      // two score tiles (slices 1-8, after the first MFMA so that block A's
      // last MFMAs have finished), the running-max decision (9), and the exp2
      // arguments (10-15).
      float mp[2][3], mh[2];
      float m_new = m_run[0];
      const float raise_above = next ? m_run[0] + kSlack : __builtin_inff();
      bool raise = false;
      auto max3f = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
      auto valu_c = [&](int c) __attribute__((always_inline)) {
        if (c >= 1 && c <= 8) {
          const int mt = (c - 1) >> 2, k = (c - 1) & 3;
          const f32x16& x = sb[mt];
          if (k == 0) { mp[mt][0] = max3f(x[0], x[1], x[2]); mp[mt][1] = max3f(x[3], x[4], x[5]); }
          if (k == 1) { mp[mt][2] = max3f(x[6], x[7], x[8]); mp[mt][0] = max3f(mp[mt][0], x[9], x[10]); }
          if (k == 2) { mp[mt][1] = max3f(mp[mt][1], x[11], x[12]); mp[mt][2] = max3f(mp[mt][2], x[13], x[14]); }
          if (k == 3) mh[mt] = fmaxf(max3f(mp[mt][0], mp[mt][1], mp[mt][2]), x[15]);
        }
        if (c == 9) {
          const float mxc = max_xor32(fmaxf(mh[0], mh[1])) * c_scale;
          raise = mxc > raise_above;  // never for the surplus tile
          m_new = raise ? mxc : m_run[0];
        }
        if (c >= 10) {
          const int i0 = (c - 10) * 32 / 6, i1 = (c - 9) * 32 / 6;
#pragma unroll
          for (int i = i0; i < i1; ++i) sb[i >> 4][i & 15] = fmaf(sb[i >> 4][i & 15], c_scale, -m_new);
        }
      };
      vread(1);
      fence();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) {
          const int slot = j * G::kOTiles + t2;
          acc[t2][0] = T::mfma32x32x16(va[j][t2], pb[j], acc[t2][0]);
          if constexpr (kSlotsC == 16) {
            valu_c(slot);
          } else {
            valu_c(2 * slot);
            valu_c(2 * slot + 1);
          }
          if (t2 == G::kOTiles - 1 && j + 2 < 4) vread(j + 2);
          fence();
        }
      }
      // The arguments are formed here, beside the MFMAs (see above).
#pragma unroll
      for (int i = 0; i < 32; ++i) asm volatile("" ::"v"(sb[i >> 4][i & 15]));
      if (__builtin_expect(__any(raise), 0)) {
        asm volatile("" ::: "memory");  // a real branch, not a speculated rescale
        rescale(m_new);
      }
      m_run[0] = m_new;
    };

    f32x16 sa[2], sb[2];
    // Prologue: tile t_begin's scores and arguments.
    scores(t_begin, sa);
    if (t_begin < t_wave_end) {
      const int jb = t_begin * kBc;
      const bool need_mask = (CAUSAL && jb + kBc - 1 > wq0 + qoff) || (jb + kBc > key_hi) ||
                             (jb < key_lo);
      if (need_mask) mask(t_begin, sa);
      float m_new;
      softmax_args(sa, true, m_new);
      m_run[0] = m_new;  // acc and l are still zero: nothing to rescale
    }
    for (int t = t_begin; t < t_end; ++t) {
      // This wave's DMAs of tile t+1 are done and its LDS reads are
      // finished; after the barrier every wave may read tile t+1, and the
      // stage of tile t-1 is free for tile t+3.
      if (t + 2 < t_end) wait_vm_lgkm0<G::kDmaPerWave>();
      else wait_vm_lgkm0<0>();
      bare_barrier();
      if (t + 3 < t_end) issue_tile(t + 3, (t + 3 - t_begin) & (kRingP - 1));
      if (t < t_wave_end) {
        step(t, sa, sb);
        sa[0] = sb[0];
        sa[1] = sb[1];
      }
    }
  }

  // -------- epilogue: O = acc / l, zero for rows without keys --------
  if constexpr (PARTIAL) {
    // float32 O of the range and lse = ln(2^m * l) (m is in log2 units); O
    // leaves through the idle ring, whole rows per store (RowStage).
    using RS = RowStage<D * 4>;
    static_assert(kWaves * kNT * RS::kBytes <= kRing * G::kStageElems * 2, "staged O fits the ring");
    wait_vm_lgkm0<0>();
    bare_barrier();  // every wave is done with the ring
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float l_tot = sum_xor32(l_run[nt]);
      const bool has = l_tot > 0.f && q_ok[nt];
      const float inv = has ? 1.f / l_tot : 0.f;
      lds_char* const ob = lds + (w * kNT + nt) * RS::kBytes;
#pragma unroll
      for (int t2 = 0; t2 < G::kOTiles; ++t2) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // columns 32 t2 + 8 g + 4 hf .. +3 of row ql
          const u32x4 x = {__float_as_uint(acc[t2][nt][4 * g] * inv),
                           __float_as_uint(acc[t2][nt][4 * g + 1] * inv),
                           __float_as_uint(acc[t2][nt][4 * g + 2] * inv),
                           __float_as_uint(acc[t2][nt][4 * g + 3] * inv)};
          RS::put(ob, ql, (32 * t2 + 8 * g + 4 * hf) * 4, x);
        }
      }
      const int r0 = wq0 + 32 * nt;
      RS::store(ob, lane, reinterpret_cast<char*>(Of + q_base + (size_t)r0 * D), (size_t)D * 4,
                n - r0);
      if (hf == 0 && qrow[nt] < n)
        Lse[q_base / D + qrow[nt]] =
            has ? (m_run[nt] + log2f(l_tot)) * kLn2 : -__builtin_inff();
    }
    return;
  }
  // Through the (now idle) K/V ring, whole rows per store (RowStage):
  // measured 3.7% faster at 2048 keys than storing from the accumulators.
  using RS = RS16;
  static_assert(kWaves * kNT * RS::kBytes <= kRing * G::kStageElems * 2, "staged O fits the ring");
  wait_vm_lgkm0<0>();
  bare_barrier();  // every wave is done with the ring
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const float l_tot = sum_xor32(l_run[nt]);
    const float inv = (l_tot > 0.f && q_ok[nt]) ? 1.f / l_tot : 0.f;
    lds_char* const ob = lds + (w * kNT + nt) * RS::kBytes;
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // columns 32 t2 + 8 g + 4 hf .. +3 of row ql
        const uint32_t lo = T::pack(acc[t2][nt][4 * g] * inv, acc[t2][nt][4 * g + 1] * inv);
        const uint32_t hi = T::pack(acc[t2][nt][4 * g + 2] * inv, acc[t2][nt][4 * g + 3] * inv);
        RS::put(ob, ql, (32 * t2 + 8 * g + 4 * hf) * 2, u32x2{lo, hi});
      }
    }
    const int r0 = wq0 + 32 * nt;
    if constexpr (kPersist) {
      static_assert(!kPersist || kNT == 1, "one pending row block per wave");
      // Held until the next unit's copies are out (or the end of the launch).
      RS::read(ob, lane, o_pend);
      o_pend_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          O + q_base + (size_t)r0 * D, 0, max(n - r0, 0) * (D * 2), (int)kRsrcWord3);
      have_pend = true;
    } else {
      RS::store(ob, lane, reinterpret_cast<char*>(O + q_base + (size_t)r0 * D), (size_t)D * 2,
                n - r0);
    }
  }
  if constexpr (!kPersist) break;  // one unit per workgroup: no loop at all
  wait_lgkm0();
  bare_barrier();  // every wave has its rows back: the next unit may refill the ring
  }  // units
  if constexpr (kPersist)
    if (have_pend) RS16::store_buf(o_pend, threadIdx.x & 63, o_pend_rsrc);
}

// ---------------------------------------------------------------------------
// float32 kernel: 16 queries per workgroup, 16 lanes per query.  Keys come in
// tiles of 16; lane j of a query scores key j of the tile in float64, the tile
// max and the weights are shared over the 16 lanes, and each lane accumulates
// D/16 output columns in float64.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 16;
constexpr int kF32Tile = 16;

// PARTIAL: keys restricted to [key_begin, key_end); also writes the natural
// log of the range's softmax denominator (Lse).  O is float32 either way.
template <int D, bool CAUSAL, bool RAGGED, bool PARTIAL>
__global__ __launch_bounds__(256) void fa_fwd_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ Lse, const int32_t* __restrict__ seq_lens, int Hq,
    int group, int n, int m, int key_begin, int key_end, int q_tiles, double scale) {
  constexpr int S = D + 1;  // padded row stride (floats) against bank conflicts
  constexpr int E = D / 16; // output columns per lane
  __shared__ float q_s[kF32Rows * S];
  __shared__ float k_s[kF32Tile * S];
  __shared__ float v_s[kF32Tile * D];

  const int tid = threadIdx.x;
  const int qi = tid >> 4, sub = tid & 15;
  const int qt = blockIdx.x % q_tiles;
  const int bh = blockIdx.x / q_tiles;
  const int b = bh / Hq, h = bh % Hq;
  const int Hkv = Hq / group;
  const float* Qh = Q + ((size_t)b * Hq + h) * (size_t)n * D;
  const float* Kh = K + ((size_t)b * Hkv + h / group) * (size_t)m * D;
  const float* Vh = V + ((size_t)b * Hkv + h / group) * (size_t)m * D;
  float* Oh = O + ((size_t)b * Hq + h) * (size_t)n * D;

  const int pad = RAGGED ? min(max(n - seq_lens[b], 0), n) : 0;
  const int q0 = qt * kF32Rows;
  const int q1 = min(n, q0 + kF32Rows);
  const int qrow = q0 + qi;
  const bool q_ok = qrow < n && qrow >= pad;

  for (int x = tid; x < kF32Rows * D; x += 256) {
    const int r = x / D, d = x % D;
    const int row = q0 + r;
    q_s[r * S + d] = (row < n && row >= pad) ? Qh[(size_t)row * D + d] : 0.f;
  }

  const int key_lo = max(RAGGED ? pad : 0, key_begin);
  const int key_hi = min(m, key_end);
  const int kv_begin = (key_lo / kF32Tile) * kF32Tile;
  const int kv_end = CAUSAL ? min(key_hi, q1) : key_hi;
  const bool no_keys = (RAGGED && q1 <= pad) || kv_end <= key_lo;
  const int t_begin = kv_begin / kF32Tile;
  const int t_end = no_keys ? t_begin : (kv_end + kF32Tile - 1) / kF32Tile;

  double m_run = -1.0e300, l_run = 0.0;
  double acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0;

  for (int t = t_begin; t < t_end; ++t) {
    const int j0 = t * kF32Tile;
    __syncthreads();
    for (int x = tid; x < kF32Tile * D; x += 256) {
      const int r = x / D, d = x % D;
      const int key = j0 + r;
      const bool ok = key < key_hi && key >= key_lo;
      k_s[r * S + d] = ok ? Kh[(size_t)key * D + d] : 0.f;
      v_s[r * D + d] = ok ? Vh[(size_t)key * D + d] : 0.f;
    }
    __syncthreads();

    const int key = j0 + sub;
    const bool ok = key < key_hi && key >= key_lo && (!CAUSAL || key <= qrow) && q_ok;
    double s = 0.0;
#pragma unroll 8
    for (int d = 0; d < D; ++d) s = fma((double)q_s[qi * S + d], (double)k_s[sub * S + d], s);
    s = ok ? s * scale : -__builtin_inf();

    double mx = s;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o, 16));
    const double m_new = fmax(m_run, mx);
    const double alpha = exp(m_run - m_new);
    const double p = ok ? exp(s - m_new) : 0.0;
    m_run = m_new;
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
    for (int jj = 0; jj < kF32Tile; ++jj) {
      const double pj = __shfl(p, jj, 16);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fma(pj, (double)v_s[jj * D + sub * E + e], acc[e]);
    }
  }

  double l_tot = l_run;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) l_tot += __shfl_xor(l_tot, o, 16);
  if (qrow < n) {
    float* orow = Oh + (size_t)qrow * D + sub * E;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = (q_ok && l_tot > 0.0) ? (float)(acc[e] / l_tot) : 0.f;
    if (PARTIAL && sub == 0)
      Lse[((size_t)b * Hq + h) * n + qrow] =
          (q_ok && l_tot > 0.0) ? (float)(m_run + log(l_tot)) : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Largest block table a paged launch stages in LDS after the K/V ring: with
// the three-stage ring, and with the pipelined loop's four-stage ring (both
// fill the 160 KB of LDS at d = 128).
constexpr int kMaxPagedBlocks = 16384;
constexpr int kMaxPipelinedPagedBlocks = 8192;

template <class T, int D, bool C, bool R, bool P, int PG>
static hipError_t launch_mfma(const FwdArgs& a) {
  using G = Geo<D>;
  const int q_tiles = (a.n + kBr - 1) / kBr;
  const long long total = (long long)a.batch * a.heads_q * q_tiles;
  const size_t ring = ring_stages(PG == 2) * G::kStageElems * sizeof(uint16_t);
  const size_t lds = PG ? ring + (size_t)a.max_blocks * sizeof(int32_t) : ring;
  const int table_max = PG == 1 ? kMaxPipelinedPagedBlocks : kMaxPagedBlocks;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa_fwd_mfma<T, D, C, R, P, PG>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(PG ? ring + table_max * sizeof(int32_t) : ring));
  if (attr != hipSuccess) return attr;
  const int bs = PG ? a.block_size : 1;
  const int shift = (PG && (bs & (bs - 1)) == 0) ? __builtin_ctz((unsigned)bs) : -1;
  // The dense non-causal form runs persistent (one workgroup per compute unit)
  // when there are at least two units per compute unit.
  long long grid = total;
  if (!C && !R && !P && PG == 0) {
    const int cus = persistent_grid();
    if (cus > 0 && total >= 2LL * cus) grid = cus;
  }
  hipLaunchKernelGGL((fa_fwd_mfma<T, D, C, R, P, PG>), dim3((unsigned)grid), dim3(kThreads), lds,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (uint16_t*)a.o, a.o_f32, a.lse, a.seq_lens,
                     a.heads_q, a.heads_q / a.heads_kv, a.n, a.m, a.key_begin, a.key_end,
                     q_tiles, (int)total, a.scale * kLog2e, a.block_table, bs, shift,
                     a.max_blocks, a.num_blocks);
  return hipGetLastError();
}

template <int D, bool C, bool R, bool P>
static hipError_t launch_f32(const FwdArgs& a) {
  const int q_tiles = (a.n + kF32Rows - 1) / kF32Rows;
  const long long total = (long long)a.batch * a.heads_q * q_tiles;
  hipLaunchKernelGGL((fa_fwd_f32<D, C, R, P>), dim3((unsigned)total), dim3(256), 0,
                     (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k,
                     (const float*)a.v, P ? a.o_f32 : (float*)a.o, a.lse, a.seq_lens, a.heads_q,
                     a.heads_q / a.heads_kv, a.n, a.m, a.key_begin, a.key_end, q_tiles,
                     (double)a.scale);
  return hipGetLastError();
}

template <class T, int D, bool P>
static hipError_t dispatch_mask(const FwdArgs& a) {
  if (a.paged) {  // paged chunks: no left padding, full key range
    if (a.max_blocks <= kMaxPipelinedPagedBlocks)
      return a.causal ? launch_mfma<T, D, true, false, false, 1>(a)
                      : launch_mfma<T, D, false, false, false, 1>(a);
    return a.causal ? launch_mfma<T, D, true, false, false, 2>(a)
                    : launch_mfma<T, D, false, false, false, 2>(a);
  }
  const bool r = a.seq_lens != nullptr;
  if (a.causal)
    return r ? launch_mfma<T, D, true, true, P, 0>(a)
             : launch_mfma<T, D, true, false, P, 0>(a);
  return r ? launch_mfma<T, D, false, true, P, 0>(a)
           : launch_mfma<T, D, false, false, P, 0>(a);
}

template <int D, bool P>
static hipError_t dispatch_f32(const FwdArgs& a) {
  const bool r = a.seq_lens != nullptr;
  if (a.causal) return r ? launch_f32<D, true, true, P>(a) : launch_f32<D, true, false, P>(a);
  return r ? launch_f32<D, false, true, P>(a) : launch_f32<D, false, false, P>(a);
}

template <bool P>
static hipError_t dispatch_dtype(const FwdArgs& a) {
  if (a.dtype == 2)
    return a.d == 128 ? dispatch_mask<BF16, 128, P>(a) : dispatch_mask<BF16, 64, P>(a);
  if (a.dtype == 1)
    return a.d == 128 ? dispatch_mask<F16, 128, P>(a) : dispatch_mask<F16, 64, P>(a);
  return a.d == 128 ? dispatch_f32<128, P>(a) : dispatch_f32<64, P>(a);
}

int max_paged_blocks() { return kMaxPagedBlocks; }

long long fwd_grid_size(int dtype, int batch, int heads_q, int n) {
  const int rows = dtype == 0 ? kF32Rows : kBr;
  return (long long)batch * heads_q * ((n + rows - 1) / rows);
}

hipError_t launch_fwd(const FwdArgs& a) {
  return a.partial ? dispatch_dtype<true>(a) : dispatch_dtype<false>(a);
}

}  // namespace fa
