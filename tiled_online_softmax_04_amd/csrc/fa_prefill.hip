// Prefill attention kernels for gfx950 (CDNA4).
//
// fa_fwd_mfma: bf16 / fp16 inputs.  One workgroup of 4 waves owns 128 query
// rows of one (batch, head); each wave owns 32 of them.  The wave keeps its
// queries resident in VGPRs as MFMA operands ("Q 常驻片上寄存器", 10100.com
// section 7) and streams 64-key K/V tiles through LDS (double-buffered, the
// next tile's global loads in flight while the current one is computed).  Per
// tile it forms S^T = K Q^T with v_mfma_f32_32x32x16, applies the online-softmax
// update of the same section (running max, rescale of the history by
// exp(m_old - m_new), running sum) and accumulates O^T += V^T P^T with a second
// MFMA.  Tiles wholly above the causal diagonal or wholly inside a left pad are
// never visited (10100.com section 6).
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

namespace fa {

// ---------------------------------------------------------------------------
// MFMA kernel geometry
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per tile
constexpr int kThreads = 64 * kWaves;

template <int D>
struct Geo {
  static constexpr int kStride = D + 8;            // K tile row stride (elements), 16 B pad
  static constexpr int kVtStride = kBc + 8;        // V^T tile row stride (elements)
  static constexpr int kKElems = kBc * kStride;
  static constexpr int kVtElems = D * kVtStride;
  static constexpr int kStage = kKElems + kVtElems;  // elements per LDS stage
  static constexpr int kChunks = D / 8;            // 16-byte chunks per row
  static constexpr int kKRowsPerPass = kThreads / kChunks;
  static constexpr int kKPasses = kBc / kKRowsPerPass;  // K chunks per thread
  static constexpr int kVKeys = D / 32;            // consecutive keys per thread (V^T)
  static constexpr int kVGroups = kBc / kVKeys;    // key groups per tile
  static constexpr int kQSteps = D / 16;           // k-steps of S^T = K Q^T
  static constexpr int kOTiles = D / 32;           // 32-row tiles of O^T
};

// Row placement of the K tile inside each 32-row block.  The accumulator of a
// 32x32x16 MFMA gives lane l, element i the row 8*(i/4) + 4*(l/32) + (i%4).
// Storing key r at LDS row kappa(r) (swap rows 4..7 with 8..11 and 20..23 with
// 24..27) makes element i of lane l hold key 16*(i/8) + 8*(l/32) + (i%8): eight
// consecutive keys per half-wave, which is exactly the B-operand layout of the
// P.V MFMA.  kappa is its own inverse.
__device__ __forceinline__ int kappa(int r) {
  return r ^ ((((r >> 2) ^ (r >> 3)) & 1) * 0xC);
}

template <class T, int D, bool CAUSAL, bool RAGGED>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, const int32_t* __restrict__ seq_lens,
    int Hq, int group, int n, int m, int q_tiles, int total, float c) {
  using G = Geo<D>;
  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ql = lane & 31, hf = lane >> 5;

  const int logical = xcd_contiguous(blockIdx.x, total);
  const int bh = logical / q_tiles;
  const int qt_ord = logical % q_tiles;
  // Causal tiles further down hold more keys: hand those out first.
  const int qt = CAUSAL ? q_tiles - 1 - qt_ord : qt_ord;
  const int b = bh / Hq, h = bh % Hq;
  const int hkv = h / group;
  const int Hkv = Hq / group;

  const size_t q_base = ((size_t)b * Hq + h) * (size_t)n * D;
  const size_t kv_base = ((size_t)b * Hkv + hkv) * (size_t)m * D;
  const uint16_t* Qh = Q + q_base;
  const uint16_t* Kh = K + kv_base;
  const uint16_t* Vh = V + kv_base;
  uint16_t* Oh = O + q_base;

  // Padding rows of a left-padded sequence; out-of-range lengths are clamped.
  const int pad = RAGGED ? min(max(n - seq_lens[b], 0), n) : 0;
  const int wg_q0 = qt * kBr;
  const int wg_q1 = min(n, wg_q0 + kBr);
  const int wq0 = wg_q0 + w * 32;  // first query of this wave
  const int qrow = wq0 + ql;       // this lane's query
  // Rows that hold no real query: past n, or inside the left pad.
  const bool q_ok = qrow < n && qrow >= pad;

  // Key range of this workgroup, in whole tiles.
  const int kv_begin = RAGGED ? (pad / kBc) * kBc : 0;
  const int kv_end = CAUSAL ? min(m, wg_q1) : m;
  const int t_begin = kv_begin / kBc;
  const int t_end = (RAGGED && wg_q1 <= pad) ? t_begin : (kv_end + kBc - 1) / kBc;

  // Queries as B operands of S^T = K Q^T: lane holds column ql, 8 consecutive d.
  u32x4 qT[G::kQSteps];
#pragma unroll
  for (int ks = 0; ks < G::kQSteps; ++ks) {
    qT[ks] = q_ok ? load16(Qh + (size_t)qrow * D + ks * 16 + hf * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc[G::kOTiles];
#pragma unroll
  for (int t = 0; t < G::kOTiles; ++t) acc[t] = f32x16{};
  float m_run = kSentinel;  // running max (scaled log2 units), finite start
  float l_run = 0.f;        // this lane's half of the running sum

  // -------- staging: global -> registers -> LDS --------
  const int kc = tid % G::kChunks, kr0 = tid / G::kChunks;
  const int vg = tid % G::kVGroups, vc = tid / G::kVGroups;
  u32x4 kreg[G::kKPasses];
  u32x4 vreg[G::kVKeys];

  auto key_valid = [&](int key) { return key < m && (!RAGGED || key >= pad); };
  auto load_tile = [&](int t) {
    const int j0 = t * kBc;
#pragma unroll
    for (int p = 0; p < G::kKPasses; ++p) {
      const int key = j0 + kr0 + p * G::kKRowsPerPass;
      kreg[p] = key_valid(key) ? load16(Kh + (size_t)key * D + kc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < G::kVKeys; ++r) {
      const int key = j0 + vg * G::kVKeys + r;
      vreg[r] = key_valid(key) ? load16(Vh + (size_t)key * D + vc * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks_ = smem + buf * G::kStage;
    uint16_t* vt_ = ks_ + G::kKElems;
#pragma unroll
    for (int p = 0; p < G::kKPasses; ++p) {
      const int r = kr0 + p * G::kKRowsPerPass;
      const int row = (r & ~31) | kappa(r & 31);
      store16(ks_ + row * G::kStride + kc * 8, kreg[p]);
    }
    // Transpose: element e of the 8 d-values of each of kVKeys keys goes to
    // V^T row vc*8+e, columns vg*kVKeys .. +kVKeys.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t wv[G::kVKeys / 2];
#pragma unroll
      for (int r2 = 0; r2 < G::kVKeys / 2; ++r2) {
        const uint32_t a = vreg[2 * r2][e >> 1], bb = vreg[2 * r2 + 1][e >> 1];
        wv[r2] = (e & 1) ? ((a >> 16) | (bb & 0xffff0000u)) : ((a & 0xffffu) | (bb << 16));
      }
      uint16_t* dst = vt_ + (vc * 8 + e) * G::kVtStride + vg * G::kVKeys;
      if constexpr (G::kVKeys == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{wv[0], wv[1]};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = wv[0];
      }
    }
  };

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) load_tile(t + 1);

    const int j0 = t * kBc;
    // Whole wave above the causal diagonal, or wholly padding: nothing to add.
    const bool wave_idle = (CAUSAL && j0 > wq0 + 31) || (RAGGED && wq0 + 31 < pad);
    if (!wave_idle) {
      const uint16_t* ks_ = smem + buf * G::kStage;
      const uint16_t* vt_ = ks_ + G::kKElems;

      // S^T[key][query] for 64 keys (two 32-row tiles) x 32 queries.
      f32x16 st0 = f32x16{}, st1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < G::kQSteps; ++ks) {
        const u32x4 a0 = load16(ks_ + ql * G::kStride + ks * 16 + hf * 8);
        const u32x4 a1 = load16(ks_ + (32 + ql) * G::kStride + ks * 16 + hf * 8);
        st0 = T::mfma32x32x16(a0, qT[ks], st0);
        st1 = T::mfma32x32x16(a1, qT[ks], st1);
      }

      // Mask only tiles that straddle the diagonal, the pad or the end of K.
      const bool need_mask = (CAUSAL && j0 + kBc - 1 > wq0) || (j0 + kBc > m) ||
                             (RAGGED && j0 < pad);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = 16 * (i >> 3) + 8 * hf + (i & 7);
          const int key0 = j0 + kk, key1 = j0 + 32 + kk;
          const bool bad0 = (CAUSAL && key0 > qrow) || key0 >= m || (RAGGED && key0 < pad);
          const bool bad1 = (CAUSAL && key1 > qrow) || key1 >= m || (RAGGED && key1 < pad);
          st0[i] = bad0 ? -__builtin_inff() : st0[i];
          st1[i] = bad1 ? -__builtin_inff() : st1[i];
        }
      }

      // Online softmax: tile row max (lane-local + partner lane 32 away).
      float mx = st0[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st0[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st1[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;

      // p = exp2(S*c - m) as the B operand of O^T += V^T P^T.
      u32x4 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * (j & 1) + 2 * e;
          const float s0 = (j < 2) ? st0[i] : st1[i];
          const float s1 = (j < 2) ? st0[i + 1] : st1[i + 1];
          const float p0 = fast_exp2(fmaf(s0, c, -m_new));
          const float p1 = fast_exp2(fmaf(s1, c, -m_new));
          psum += p0 + p1;
          pb[j][e] = T::pack(p0, p1);
        }
      }
      l_run = fmaf(l_run, alpha, psum);

#pragma unroll
      for (int t2 = 0; t2 < G::kOTiles; ++t2) acc[t2] *= alpha;

#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t2 = 0; t2 < G::kOTiles; ++t2) {
          const u32x4 a = load16(vt_ + (32 * t2 + ql) * G::kVtStride + 16 * j + 8 * hf);
          acc[t2] = T::mfma32x32x16(a, pb[j], acc[t2]);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // -------- epilogue: O = acc / l, zero for rows without keys --------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = (l_tot > 0.f && q_ok) ? 1.f / l_tot : 0.f;
  if (qrow < n && qrow >= wg_q0) {
    uint16_t* orow = Oh + (size_t)qrow * D;
#pragma unroll
    for (int t2 = 0; t2 < G::kOTiles; ++t2) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dv0 = 32 * t2 + 8 * g + 4 * hf;
        const uint32_t lo = T::pack(acc[t2][4 * g] * inv, acc[t2][4 * g + 1] * inv);
        const uint32_t hi = T::pack(acc[t2][4 * g + 2] * inv, acc[t2][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dv0) = u32x2{lo, hi};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 kernel: 16 queries per workgroup, 16 lanes per query.  Keys come in
// tiles of 16; lane j of a query scores key j of the tile in float64, the tile
// max and the weights are shared over the 16 lanes, and each lane accumulates
// D/16 output columns in float64.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 16;
constexpr int kF32Tile = 16;

template <int D, bool CAUSAL, bool RAGGED>
__global__ __launch_bounds__(256) void fa_fwd_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, const int32_t* __restrict__ seq_lens, int Hq, int group, int n, int m,
    int q_tiles, double scale) {
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

  const int kv_begin = RAGGED ? (pad / kF32Tile) * kF32Tile : 0;
  const int kv_end = CAUSAL ? min(m, q1) : m;
  const int t_begin = kv_begin / kF32Tile;
  const int t_end = (RAGGED && q1 <= pad) ? t_begin : (kv_end + kF32Tile - 1) / kF32Tile;

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
      const bool ok = key < m && key >= pad;
      k_s[r * S + d] = ok ? Kh[(size_t)key * D + d] : 0.f;
      v_s[r * D + d] = ok ? Vh[(size_t)key * D + d] : 0.f;
    }
    __syncthreads();

    const int key = j0 + sub;
    const bool ok = key < m && key >= pad && (!CAUSAL || key <= qrow) && q_ok;
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
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <class T, int D, bool C, bool R>
static hipError_t launch_mfma(const FwdArgs& a) {
  using G = Geo<D>;
  const int q_tiles = (a.n + kBr - 1) / kBr;
  const long long total = (long long)a.batch * a.heads_q * q_tiles;
  const size_t lds = 2 * G::kStage * sizeof(uint16_t);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fa_fwd_mfma<T, D, C, R>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fa_fwd_mfma<T, D, C, R>), dim3((unsigned)total), dim3(kThreads), lds,
                     (hipStream_t)a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (uint16_t*)a.o, a.seq_lens, a.heads_q,
                     a.heads_q / a.heads_kv, a.n, a.m, q_tiles, (int)total,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool C, bool R>
static hipError_t launch_f32(const FwdArgs& a) {
  const int q_tiles = (a.n + kF32Rows - 1) / kF32Rows;
  const long long total = (long long)a.batch * a.heads_q * q_tiles;
  hipLaunchKernelGGL((fa_fwd_f32<D, C, R>), dim3((unsigned)total), dim3(256), 0,
                     (hipStream_t)a.stream, (const float*)a.q, (const float*)a.k,
                     (const float*)a.v, (float*)a.o, a.seq_lens, a.heads_q,
                     a.heads_q / a.heads_kv, a.n, a.m, q_tiles, (double)a.scale);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t dispatch_mask(const FwdArgs& a) {
  const bool r = a.seq_lens != nullptr;
  if (a.causal) return r ? launch_mfma<T, D, true, true>(a) : launch_mfma<T, D, true, false>(a);
  return r ? launch_mfma<T, D, false, true>(a) : launch_mfma<T, D, false, false>(a);
}

template <int D>
static hipError_t dispatch_f32(const FwdArgs& a) {
  const bool r = a.seq_lens != nullptr;
  if (a.causal) return r ? launch_f32<D, true, true>(a) : launch_f32<D, true, false>(a);
  return r ? launch_f32<D, false, true>(a) : launch_f32<D, false, false>(a);
}

long long fwd_grid_size(int dtype, int batch, int heads_q, int n) {
  const int rows = dtype == 0 ? kF32Rows : kBr;
  return (long long)batch * heads_q * ((n + rows - 1) / rows);
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == 2) return a.d == 128 ? dispatch_mask<BF16, 128>(a) : dispatch_mask<BF16, 64>(a);
  if (a.dtype == 1) return a.d == 128 ? dispatch_mask<F16, 128>(a) : dispatch_mask<F16, 64>(a);
  return a.d == 128 ? dispatch_f32<128>(a) : dispatch_f32<64>(a);
}

}  // namespace fa
