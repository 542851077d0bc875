// Device helpers of the indexer kernels: pooling of one block, the
// per-row query side of the indexer score and the chunked score stream
// (shared by the score, pooling and top-k kernels).
#pragma once

#include <type_traits>

#include "index.hpp"

namespace qsa {

// ================================================================ pooling

// Lane `part` (of Di / V) of the pooled key of block b of sequence s: the
// mean of the block's indexer keys, summed in float32 in token order.
template <typename T, int DI>
__device__ __forceinline__ void pool_part(const PageMap& pm, const T* kidx, T* kbar, int s,
                                          int b, int part) {
  constexpr int V = Vec<T>::N;
  const int nb = 1 << pm.blk_shift;
  const int64_t row0 = pm.token_slot(s, b << pm.blk_shift);  // nb rows, one page
  const T* src = kidx + row0 * DI + part * V;
  float o[V];
  if (nb == 4) {  // QSA: all four loads in flight at once
    float r0[V], r1[V], r2[V], r3[V];
    Vec<T>::load(src, r0);
    Vec<T>::load(src + DI, r1);
    Vec<T>::load(src + 2 * DI, r2);
    Vec<T>::load(src + 3 * DI, r3);
#pragma unroll
    for (int i = 0; i < V; ++i) o[i] = ((r0[i] + r1[i]) + r2[i]) + r3[i];
  } else {
    Vec<T>::load(src, o);
    for (int j = 1; j < nb; ++j) {
      float r[V];
      Vec<T>::load(src + j * DI, r);
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] += r[i];
    }
  }
  // the mean: a power-of-two scale, exact
  const float inv = 1.0f / (float)nb;
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] *= inv;
  Vec<T>::store(kbar + pm.block_slot(s, b) * DI + part * V, o);
}

// ================================================================ scores

// Per-thread slice of one query row's indexer: this lane's V dims of each of
// the HI heads (heads beyond the real count have zero weight), and weights.
template <typename T, int DI, int HI>
struct IdxQuery {
  static constexpr int V = Vec<T>::N;
  static constexpr int G = DI / V;
  float q[HI][V];
  float w[HI];
  __device__ __forceinline__ void load(const T* q_idx_row, const float* w_row, int hi,
                                       int part) {
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      if (h < hi) {
        Vec<T>::load(q_idx_row + h * DI + part * V, q[h]);
        w[h] = w_row[h];
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) q[h][i] = 0.0f;
        w[h] = 0.0f;
      }
    }
  }
  // score of the row whose V-slice this lane holds in x; all G lanes of the
  // group return the same value
  __device__ __forceinline__ float score(const float (&x)[V]) const {
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) acc = fmaf(q[h][i], x[i], acc);
      acc = group_sum<G>(acc);
      s = fmaf(w[h], fmaxf(acc, 0.0f), s);
    }
    return canon_zero(s);
  }
};

// bfloat16 rows: G = Di / 16 lanes per pooled key, each holding two
// 16-byte pieces of it -- dims [8p, 8p + 8) and [8(p + G), 8(p + G) + 8) of
// lane p of the group, so each of the two loads of a group reads one
// contiguous half of the row.  Dot products use v_dot2_f32_bf16 on packed
// pairs (products exact in fp32, accumulated in fp32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int DI, int HI>
struct IdxQueryBf16 {
  static constexpr int G = DI / 16;
  uint32_t q[HI][8];
  float w[HI];
  __device__ __forceinline__ void load(const bf16_t* q_idx_row, const float* w_row, int hi,
                                       int part) {
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
      w[h] = 0.0f;
      if (h < hi) {
        a = *reinterpret_cast<const uint4*>(q_idx_row + h * DI + 8 * part);
        b = *reinterpret_cast<const uint4*>(q_idx_row + h * DI + 8 * (part + G));
        w[h] = w_row[h];
      }
      q[h][0] = a.x; q[h][1] = a.y; q[h][2] = a.z; q[h][3] = a.w;
      q[h][4] = b.x; q[h][5] = b.y; q[h][6] = b.z; q[h][7] = b.w;
    }
  }
  __device__ __forceinline__ float score(const uint4& x0, const uint4& x1) const {
    const uint32_t x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < HI; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = dot2_bf16(q[h][i], x[i], acc);
      acc = group_sum<G>(acc);
      s = fmaf(w[h], fmaxf(acc, 0.0f), s);
    }
    return canon_zero(s);
  }
};

__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Page ids of the blocks [c0, c0 + kChunk) of sequence seq, staged in LDS.
__device__ __forceinline__ void stage_pages(const PageMap& pm, int seq, int c0, int n,
                                            int32_t* pages) {
  const int first = c0 >> pm.bpp_shift();
  const int last_b = min(c0 + kChunk, n) - 1;
  const int cnt = (last_b >> pm.bpp_shift()) - first + 1;
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) pages[i] = pm.page(seq, first + i);
  __syncthreads();
}

// Query side of one row for element type T: fp32 rows use IdxQuery,
// bfloat16 rows the packed-pair IdxQueryBf16.
template <typename T, int DI, int HI>
struct RowQuery {
  using type = IdxQuery<T, DI, HI>;
  static constexpr int G = type::G;
};
template <int DI, int HI>
struct RowQuery<bf16_t, DI, HI> {
  using type = IdxQueryBf16<DI, HI>;
  static constexpr int G = type::G;
};

template <typename T, int DI, int HI>
__device__ __forceinline__ void load_row_query(typename RowQuery<T, DI, HI>::type& iq,
                                               const IdxArgs& a, int row) {
  iq.load(static_cast<const T*>(a.q_idx) + (int64_t)row * a.hi * DI, a.w + (int64_t)row * a.hi,
          a.hi, threadIdx.x % RowQuery<T, DI, HI>::G);
}

// Scores of blocks [c0, c0 + kChunk) of one row, computed by the whole
// workgroup into keys[] (ordered keys; blocks >= n get key 0).  All of a
// thread's loads of a pass are issued before any is used.
template <typename T, int DI, int HI>
__device__ __forceinline__ void chunk_scores(const IdxArgs& a, int seq, int n, int c0,
                             const typename RowQuery<T, DI, HI>::type& iq, int32_t* pages,
                             uint32_t* keys) {
  constexpr bool kBf = std::is_same<T, bf16_t>::value;
  constexpr int G = RowQuery<T, DI, HI>::G;
  constexpr int LPR = kBf ? 2 : 1;        // 16-byte loads per lane per row
  constexpr int RPI = 256 / G;            // rows per workgroup iteration
  constexpr int NIT = kChunk / RPI;       // iterations per chunk
  constexpr int U = NIT * LPR < 32 ? NIT : 32 / LPR;  // iterations in flight
  stage_pages(a.pm, seq, c0, n, pages);
  const T* kbar = static_cast<const T*>(a.kbar);
  const int gi = threadIdx.x / G, part = threadIdx.x % G;
  const int bsh = a.pm.bpp_shift();  // log2(blocks per page)
  const int first = c0 >> bsh;
#pragma unroll 1
  for (int it0 = 0; it0 < NIT; it0 += U) {
    uint4 raw[U][LPR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = c0 + (it0 + u) * RPI + gi;
      if (b < n) {
        const int64_t slot =
            ((int64_t)pages[(b >> bsh) - first] << bsh) +
            (b & ((1 << bsh) - 1));
        const T* rowp = kbar + slot * DI;
        if constexpr (kBf) {
          raw[u][0] = *reinterpret_cast<const uint4*>(rowp + 8 * part);
          raw[u][LPR - 1] = *reinterpret_cast<const uint4*>(rowp + 8 * (part + G));
        } else {
          raw[u][0] = *reinterpret_cast<const uint4*>(rowp + 4 * part);
        }
      } else {
#pragma unroll
        for (int j = 0; j < LPR; ++j) raw[u][j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s;
      if constexpr (kBf) {
        s = iq.score(raw[u][0], raw[u][LPR - 1]);
      } else {
        float x[4] = {__uint_as_float(raw[u][0].x), __uint_as_float(raw[u][0].y),
                      __uint_as_float(raw[u][0].z), __uint_as_float(raw[u][0].w)};
        s = iq.score(x);
      }
      const int i = (it0 + u) * RPI + gi;
      if (part == 0) keys[i] = (c0 + i < n) ? score_key(s) : 0u;
    }
  }
  __syncthreads();
}

// Keys of the kRun blocks [b0, b0 + kRun) of one row, computed by the
// calling wave alone into dst[0, kRun) (blocks >= n get key 0).  The lane
// layout (G lanes per block, lane part = lane % G holding the same slice of
// the query as in chunk_scores) and the arithmetic are chunk_scores', so
// each key equals the one the chunked pass computed, bit for bit.  The
// wave's own later LDS reads see dst; other waves need a barrier.
constexpr int kRun = 256;
template <typename T, int DI, int HI>
__device__ __forceinline__ void run_scores(const IdxArgs& a, int seq, int n, int b0,
                                           const typename RowQuery<T, DI, HI>::type& iq,
                                           uint32_t* dst) {
  constexpr bool kBf = std::is_same<T, bf16_t>::value;
  constexpr int G = RowQuery<T, DI, HI>::G;
  static_assert(kWave % G == 0, "a block's lanes lie in one wave");
  constexpr int LPR = kBf ? 2 : 1;
  constexpr int RPW = kWave / G;          // blocks per wave iteration
  constexpr int NIT = kRun / RPW;
  constexpr int U = NIT * LPR < 32 ? NIT : 32 / LPR;
  const T* kbar = static_cast<const T*>(a.kbar);
  const int lane = lane_id(), gi = lane / G, part = lane % G;
#pragma unroll 1
  for (int it0 = 0; it0 < NIT; it0 += U) {
    uint4 raw[U][LPR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = b0 + (it0 + u) * RPW + gi;
      if (b < n) {
        const T* rowp = kbar + a.pm.block_slot(seq, b) * DI;
        if constexpr (kBf) {
          raw[u][0] = *reinterpret_cast<const uint4*>(rowp + 8 * part);
          raw[u][LPR - 1] = *reinterpret_cast<const uint4*>(rowp + 8 * (part + G));
        } else {
          raw[u][0] = *reinterpret_cast<const uint4*>(rowp + 4 * part);
        }
      } else {
#pragma unroll
        for (int j = 0; j < LPR; ++j) raw[u][j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s;
      if constexpr (kBf) {
        s = iq.score(raw[u][0], raw[u][LPR - 1]);
      } else {
        float x[4] = {__uint_as_float(raw[u][0].x), __uint_as_float(raw[u][0].y),
                      __uint_as_float(raw[u][0].z), __uint_as_float(raw[u][0].w)};
        s = iq.score(x);
      }
      const int i = (it0 + u) * RPW + gi;
      if (part == 0) dst[i] = (b0 + i < n) ? score_key(s) : 0u;
    }
  }
  // the wave's LDS operations complete in order; keep the compiler from
  // moving the callers' reads above these writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace qsa
