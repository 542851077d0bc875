// Indexer side of the QSA hot path on gfx950: block pooling, block scores
// and the exact per-query top-k block selection.
//
//   pooling    -- keieiax.jp glossary "Qwen Sparse Attention", section
//                 4トークンずつまとめて: the context is compressed into 4-token
//                 micro-blocks; blog.cecily.jp/6295 (PR #30965 digest), the
//                 paragraph on Raschka's explanation: keys are averaged per
//                 block.
//   scores     -- same passages: a learned lightweight indexer rates every
//                 block; the rating used here is
//                 s[b] = sum_h w[h] * max(0, q_idx[h] . kbar[b]).
//   selection  -- same glossary section: at most 512 blocks per query, best
//                 first; ties go to the lower block id and the ids are
//                 reported in ascending order.
//
// Streaming layout: a pooled key row is Di elements (128 B for 64 bf16);
// G = Di / (16 B of elements) lanes cooperate on one row so each load
// instruction reads whole rows, fully coalesced, and the per-row dot
// products are summed across the G lanes with DPP.  A workgroup owns a chunk
// of kChunk consecutive blocks of one query row: it first stages the
// chunk's page ids in LDS, then issues every pooled-key load of the chunk
// before using any, so one round trip to memory covers the whole chunk.
#include <type_traits>

#include "index.hpp"
#include "select.hpp"

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

template <typename T, int DI>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  constexpr int G = DI / Vec<T>::N;  // lanes per block row
  const int s = blockIdx.y;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int bl = gid / G, part = gid % G;
  if (bl >= a.max_new) return;
  const int b0 = a.blk_begin[s];
  const int b = (b0 < 0 ? 0 : b0) + bl;
  const int len = min(a.seq_len[s], a.max_seq_len);
  if (b >= (len >> a.pm.blk_shift)) return;
  pool_part<T, DI>(a.pm, static_cast<const T*>(a.kidx), static_cast<T*>(a.kbar), s, b, part);
}

// The newest complete block before each row's position (block pos/B - 1 of
// its sequence), pooled per row: one workgroup of Di / V lanes per row.
template <typename T, int DI>
__global__ void __launch_bounds__(64) pool_rows_kernel(IdxArgs a, const void* kidx) {
  constexpr int G = DI / Vec<T>::N;
  const int row = blockIdx.x;
  const int n = a.pos_of(row) >> a.pm.blk_shift;
  if (threadIdx.x >= G || n < 1) return;
  pool_part<T, DI>(a.pm, static_cast<const T*>(kidx),
                   static_cast<T*>(const_cast<void*>(a.kbar)), a.seq_of(row), n - 1,
                   threadIdx.x);
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
  const int32_t* row = pm.table + (int64_t)seq * pm.max_pages + first;
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) pages[i] = row[i];
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

template <typename T, int DI, int HI>
__global__ void __launch_bounds__(256) scores_kernel(IdxArgs a, float* scores, int64_t ld) {
  __shared__ uint32_t keys[kChunk];
  __shared__ int32_t pages[kChunk];
  const int row = blockIdx.y;
  const int seq = a.seq_of(row);
  const int n = a.pos_of(row) >> a.pm.blk_shift;
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= n) return;
  typename RowQuery<T, DI, HI>::type iq;
  load_row_query<T, DI, HI>(iq, a, row);
  chunk_scores<T, DI, HI>(a, seq, n, c0, iq, pages, keys);
  float* out = scores + (int64_t)row * ld + c0;
  for (int i = threadIdx.x; i < kChunk && c0 + i < n; i += blockDim.x)
    out[i] = key_to_score(keys[i]);
}

// ================================================================ top-k

// Per-row plan.
struct RowPlan {
  int seq, n, W, jw;
  __device__ __forceinline__ RowPlan(const TopkArgs& t, int row) {
    seq = t.idx.seq_of(row);
    n = t.idx.pos_of(row) >> t.idx.pm.blk_shift;
    W = (n + kChunk - 1) / kChunk;
    jw = row_jw(n, t.ucap);
  }
};

struct SelfId {
  __device__ __forceinline__ int32_t operator()(int e) const { return e; }
};
struct KeyArray {  // keys in LDS or global memory
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int e) const { return k[e]; }
};
struct ScoreKeys {  // keys of caller scores
  const float* s;
  __device__ __forceinline__ uint32_t operator()(int e) const { return score_key(s[e]); }
};
struct IdArray {
  const int32_t* id;
  __device__ __forceinline__ int32_t operator()(int e) const { return id[e]; }
};

// Key of candidate e of a row from whichever source the row has: caller
// scores, keys stored in the workspace, or (rare exact fallback of rows
// whose keys are not stored) recomputed by this lane alone.
template <typename T, int DI>
struct RowKeys {
  const float* given;
  const uint32_t* stored;
  const T* kbar;
  const T* qrow;     // the row's q_idx, [hi][DI]
  const float* wrow; // the row's head weights
  const int32_t* pages;  // the sequence's row of the page table
  int hi, bsh;           // heads; log2(blocks per page)
  // (56 bytes: small enough to travel in registers to the out-of-line
  // selection routines)
  __device__ __forceinline__ RowKeys(const float* g, const uint32_t* st, const TopkArgs& t, int row,
                                     int sq)
      : given(g), stored(st), kbar(static_cast<const T*>(t.idx.kbar)),
        qrow(static_cast<const T*>(t.idx.q_idx) + (int64_t)row * t.idx.hi * DI),
        wrow(t.idx.w + (int64_t)row * t.idx.hi),
        pages(t.idx.pm.table + (int64_t)sq * t.idx.pm.max_pages), hi(t.idx.hi),
        bsh(t.idx.pm.bpp_shift()) {}
  __device__ __forceinline__ uint32_t operator()(int e) const {
    if (given != nullptr) return score_key(given[e]);
    if (stored != nullptr) return stored[e];
    const int64_t slot = ((int64_t)pages[e >> bsh] << bsh) + (e & ((1 << bsh) - 1));
    const T* p = kbar + slot * DI;
    float s = 0.0f;
    for (int h = 0; h < hi; ++h) {
      float d = 0.0f;
      for (int c = 0; c < DI; ++c) d = fmaf(to_f32(qrow[h * DI + c]), to_f32(p[c]), d);
      s = fmaf(wrow[h], fmaxf(d, 0.0f), s);
    }
    return score_key(s);
  }
};

__device__ __forceinline__ void write_all(int32_t* sel_row, int32_t* n_sel, int row, int n,
                                          int top_k) {
  for (int j = threadIdx.x; j < top_k; j += blockDim.x) sel_row[j] = j < n ? j : -1;
  if (threadIdx.x == 0) n_sel[row] = n;
}

// Exact selection over every candidate of a row straight from a key source.
template <class Get>
__device__ __noinline__ void select_full(Get get, int n, int top_k, int32_t* sel_row, int32_t* n_sel,
                            int row, SelShared& sh) {
  uint32_t thr;
  int r;
  radix_kth(get, n, top_k, sh, thr, r);
  emit_topk(get, SelfId{}, n, thr, r, sel_row, top_k, sh);
  if (threadIdx.x == 0) n_sel[row] = top_k;
}

// One workgroup per (row, chunk of kChunk candidates).
//
// Rows with at most kDirectCap candidates: the chunks store their keys; the
// last chunk of the row to finish selects over all of them in LDS.
//
// Longer rows: each of the chunk's four waves publishes its jw largest
// (key, id) pairs.  The last chunk takes tau = the k-th largest key of all
// published pairs: tau is a key of the row, and at least k keys are >= tau,
// so tau never exceeds the row's k-th largest key and every selected block
// has key >= tau.  A wave whose jw-th published key is below tau has all of
// its keys >= tau among its published pairs; only a wave whose jw-th key
// reaches tau ("saturated", rare) is rescanned.  The survivors are gathered
// wave by wave, ascending ids inside each wave, so they come out in
// ascending id order, and the exact radix select + ordered emission of
// select.hpp picks the k best with ties to the lower id.
constexpr int kMaxSat = 64;  // saturated waves rescanned per row (else exact fallback)
constexpr int kWaveSel = 16;  // survivors per lane of the one-wave final select (1,024)

// LDS of the tail of a long row.
struct LongShared {
  uint32_t skey[kSelCap];  // survivors, in ascending id order
  int32_t sid[kSelCap];
  int32_t sat_w[kMaxSat];  // saturated runs
  uint32_t sat_cnt[kMaxSat], sat_off[kMaxSat];
  uint32_t n_sat;
};

// Tail of a long row (the last chunk to finish), JW keys per published run.
// Thread t holds union entries [E t, E t + E) -- whole runs, E = union cap /
// 256 -- in registers, loaded at once.  tau = the k-th largest union key
// (low bits past two radix digits cleared); a run whose last published key
// reaches tau is saturated and rescanned from the key source; the other
// runs' survivors (key >= tau) are placed in id order straight from the
// registers, each run's entries ranked by id (a run lists one wave's keys
// best first).  Then the exact select among the survivors.
template <int JW, int E, class Src>
__device__ __forceinline__ void long_tail(const Src& src, const uint64_t* tops, int nw, int n,
                                          int top_k, int32_t* sel_row, int32_t* n_sel, int row,
                                          LongShared& ls, SelShared& sh) {
  static_assert(JW <= E, "a thread holds whole runs");
  constexpr int R = E / JW;
  const int un = nw * JW;
  const int e0 = (int)threadIdx.x * E;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  uint32_t k[E];
  int32_t id[E];
  {
    uint64_t v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = e0 + i < un ? tops[e0 + i] : 0ull;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      k[i] = (uint32_t)v[i];
      id[i] = (int32_t)(v[i] >> 32);
    }
  }
  if (threadIdx.x == 0) ls.n_sat = 0u;
  uint32_t tau = 1u;  // a union smaller than top_k bounds nothing: every key survives
  if (un >= top_k) {
    int r;
    bool resolved;
    radix_kth_regs<E>(k, un, top_k, sh, tau, r, resolved, 2);
  }
  // saturated runs (index into sat_w, or 0xff)
  int si[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    si[rr] = 0xff;
    const uint32_t last = k[rr * JW + JW - 1];
    if (e0 + rr * JW < un && last >= tau && last != 0u) {
      const uint32_t sidx = atomicAdd(&ls.n_sat, 1u);
      if (sidx < (uint32_t)kMaxSat) {
        ls.sat_w[sidx] = e0 / JW + rr;
        si[rr] = (int)sidx;
      }
    }
  }
  __syncthreads();
  const int ns = (int)ls.n_sat;
  bool fits = ns <= kMaxSat;
  // survivor counts of saturated runs (a run is one scoring wave's 256
  // candidates; wave w of this workgroup counts runs w, w + 4, ..., its
  // lanes reading 4 keys each, with no workgroup barrier per run)
#pragma unroll 1
  for (int i = wave; fits && i < ns; i += kSelWaves) {
    const int e0 = ls.sat_w[i] * 256 + lane;
    uint32_t cw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 64 * j;
      cw += (uint32_t)__popcll(ballot(e < n && src(e) >= tau));
    }
    if (lane == 0) ls.sat_cnt[i] = cw;
  }
  __syncthreads();
  // survivors of the unsaturated runs placed, saturated runs' places reserved
  uint32_t cnt[R], mine = 0;
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < JW; ++j) c += (k[rr * JW + j] >= tau && k[rr * JW + j] != 0u) ? 1u : 0u;
    cnt[rr] = si[rr] != 0xff ? ls.sat_cnt[si[rr]] : c;
    mine += cnt[rr];
  }
  uint32_t m_total;
  uint32_t off = block_incl_scan(mine, sh, m_total) - mine;
  fits = fits && m_total <= (uint32_t)kSelCap;
  if (fits) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      if (si[rr] != 0xff) {
        ls.sat_off[si[rr]] = off;
      } else {
#pragma unroll
        for (int i = 0; i < JW; ++i) {
          const uint32_t ki = k[rr * JW + i];
          if (ki >= tau && ki != 0u) {
            uint32_t rank = 0;
#pragma unroll
            for (int j = 0; j < JW; ++j) {
              const uint32_t kj = k[rr * JW + j];
              rank += (kj >= tau && kj != 0u && id[rr * JW + j] < id[rr * JW + i]) ? 1u : 0u;
            }
            ls.skey[off + rank] = ki;
            ls.sid[off + rank] = id[rr * JW + i];
          }
        }
      }
      off += cnt[rr];
    }
  }
  __syncthreads();
  // survivors of saturated runs, in id order (wave w places runs w, w + 4,
  // ...; a run's ids ascend with 64 j + lane)
#pragma unroll 1
  for (int i = wave; fits && i < ns; i += kSelWaves) {
    const int e0 = ls.sat_w[i] * 256 + lane;
    uint32_t base = ls.sat_off[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 64 * j;
      const uint32_t kk = e < n ? src(e) : 0u;
      const bool hit = e < n && kk >= tau;
      const uint64_t m = ballot(hit);
      if (hit) {
        ls.skey[base + lanes_below(m)] = kk;
        ls.sid[base + lanes_below(m)] = e;
      }
      base += (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  if (fits && m_total == (uint32_t)top_k) {
    // exactly k survivors: all of them, already in id order
    for (int j = threadIdx.x; j < top_k; j += kSelThreads) sel_row[j] = ls.sid[j];
    if (threadIdx.x == 0) n_sel[row] = top_k;
  } else if (fits && m_total <= (uint32_t)(kWave * kWaveSel)) {
    // few survivors: one wave selects them (element jj at lane jj % 64)
    if (wave == 0) {
      uint32_t key[kWaveSel];
      int32_t sid[kWaveSel];
#pragma unroll
      for (int i = 0; i < kWaveSel; ++i) {
        const uint32_t jj = (uint32_t)(i * kWave + lane);
        key[i] = jj < m_total ? ls.skey[jj] : 0u;
        sid[i] = jj < m_total ? ls.sid[jj] : 0;
      }
      wave_topk_ordered<kWaveSel>(key, sid, top_k, sel_row);
      if (lane == 0) n_sel[row] = top_k;
    }
  } else if (fits) {
    uint32_t thr;
    int r;
    radix_kth(KeyArray{ls.skey}, (int)m_total, top_k, sh, thr, r);
    emit_topk(KeyArray{ls.skey}, IdArray{ls.sid}, (int)m_total, thr, r, sel_row, top_k, sh);
    if (threadIdx.x == 0) n_sel[row] = top_k;
  } else {
    // rare: too many survivors (heavy ties): exact select over every key
    select_full(src, n, top_k, sel_row, n_sel, row, sh);
  }
}

// Exact top-k of a row of n <= kDirectCap candidates whose keys get(e)
// returns: thread t holds keys t * EPT .. t * EPT + EPT - 1 in registers
// (all of its loads in flight at once), then a register radix select and
// ordered emission.  Kept out of line: it runs once per row.
template <class Get>
__device__ __noinline__ void select_direct(Get get, int n, int top_k, int32_t* sel_row,
                                           int32_t* n_sel, int row, SelShared& sh) {
  constexpr int EPT = kDirectCap / kSelThreads;
  const int base = (int)threadIdx.x * EPT;
  uint32_t key[EPT];
  int32_t id[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    key[i] = get(min(base + i, n - 1));
    id[i] = base + i;
  }
  uint32_t thr;
  int r;
  bool resolved;
  radix_kth_regs<EPT>(key, n, top_k, sh, thr, r, resolved);
  emit_regs<EPT>(key, id, n, thr, r, sel_row, top_k, sh);
  if (threadIdx.x == 0) n_sel[row] = top_k;
}

// UCAP: the union capacity of the call.  With kUnionCapL the tail of the
// long rows runs in topk_tail_kernel (64 union entries per thread would
// crowd this kernel's registers).
template <typename T, int DI, int HI, int UCAP>
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs t) {
  __shared__ uint32_t keys[kChunk];
  __shared__ int32_t pages[kChunk];
  __shared__ LongShared ls;
  __shared__ SelShared sh;
  __shared__ uint32_t flag;
  const int rl = blockIdx.y, row = t.row0 + rl, c = blockIdx.x;
  const RowPlan p(t, row);
  if (t.pool_kidx != nullptr && p.n >= 1 && c == (p.n - 1) / kChunk) {
    // the row's newest complete block, pooled by the workgroup whose chunk
    // scores it, before the scores: published with an agent-scope release
    // so that the row's tail, in whichever workgroup arrives last, reads it
    constexpr int G = DI / Vec<T>::N;
    if (threadIdx.x < G) {
      pool_part<T, DI>(t.idx.pm, static_cast<const T*>(t.pool_kidx),
                       static_cast<T*>(const_cast<void*>(t.idx.kbar)), p.seq, p.n - 1,
                       threadIdx.x);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    __syncthreads();
  }
  int32_t* sel_row = t.sel + (int64_t)row * t.top_k;
  if (p.n <= t.top_k) {
    if (c == 0) write_all(sel_row, t.n_sel, row, p.n, t.top_k);
    return;
  }
  const bool direct = p.n <= kDirectCap;
  const float* given = t.scores ? t.scores + (int64_t)row * t.ld : nullptr;
  if (direct && given) {  // every score is stored already: one workgroup
    if (c != 0) return;
    select_direct(ScoreKeys{given}, p.n, t.top_k, sel_row, t.n_sel, row, sh);
    return;
  }
  if (c >= p.W) return;
  const int c0 = c * kChunk;
  uint32_t* ws_row = reinterpret_cast<uint32_t*>(t.ws_scores + (int64_t)rl * t.ws_ld);
  const bool keep = !given && (direct || t.materialize);
  if (given) {
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x)
      keys[i] = (c0 + i < p.n) ? score_key(given[c0 + i]) : 0u;
    __syncthreads();
  } else {
    typename RowQuery<T, DI, HI>::type iq;
    load_row_query<T, DI, HI>(iq, t.idx, row);
    chunk_scores<T, DI, HI>(t.idx, p.seq, p.n, c0, iq, pages, keys);
    if (keep) {
      for (int i = threadIdx.x; i < kChunk && c0 + i < p.n; i += blockDim.x)
        st_agent(ws_row + c0 + i, keys[i]);
    }
  }
  constexpr bool OWN_TAIL = UCAP <= kUnionCapM;  // the tail runs here
  uint64_t* tops = t.tops + (int64_t)rl * UCAP;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  if (!direct) {
    // per-wave top-jw (key, id) pairs of this chunk, best first (key 0 =
    // nothing left)
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = keys[wave * 256 + lane + 64 * i];
    uint64_t* dst = tops + (c * kSelWaves + wave) * p.jw;
    for (int j = 0; j < p.jw; ++j) {
      const uint32_t lm = max(max(v[0], v[1]), max(v[2], v[3]));
      const uint32_t wm = wave_max_u32(lm);
      const uint64_t b = ballot(lm == wm);
      if (lane == (int)(__ffsll((unsigned long long)b) - 1)) {
        int hit = 0;
#pragma unroll
        for (int i = 3; i >= 0; --i)
          if (v[i] == wm) hit = i;
        const uint32_t id = (uint32_t)(c0 + wave * 256 + lane + 64 * hit);
        st_agent(dst + j, ((uint64_t)id << 32) | wm);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i == hit) v[i] = 0u;
      }
    }
  }
  if (!OWN_TAIL && !direct) return;  // the tail follows in topk_tail_kernel
  if (!arrive_last(t.cnt + rl, (uint32_t)p.W, &flag)) return;
  if (direct) {
    select_direct(KeyArray{ws_row}, p.n, t.top_k, sel_row, t.n_sel, row, sh);
    return;
  }

  // ---- last chunk of a long row
  if constexpr (OWN_TAIL) {
    const RowKeys<T, DI> src(given, keep ? ws_row : nullptr, t, row, p.seq);
    const int nw = p.W * kSelWaves;
    constexpr int E = UCAP / kSelThreads;
    switch (p.jw) {
      case 1: long_tail<1, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
      case 2: long_tail<2, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
      case 4: long_tail<4, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
      case 8: long_tail<8, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
      case 16: long_tail<16, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
      default:
        if constexpr (E >= 32)
          long_tail<32, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh);
        break;
    }
  }
}

// The tail of the long rows of a large selection, after topk_kernel has
// published every chunk's per-wave tops: one workgroup per row.
template <typename T, int DI>
__global__ void __launch_bounds__(256) topk_tail_kernel(TopkArgs t) {
  __shared__ LongShared ls;
  __shared__ SelShared sh;
  const int rl = blockIdx.x, row = t.row0 + rl;
  const RowPlan p(t, row);
  if (p.n <= t.top_k || p.n <= kDirectCap) return;  // done by topk_kernel
  int32_t* sel_row = t.sel + (int64_t)row * t.top_k;
  const float* given = t.scores ? t.scores + (int64_t)row * t.ld : nullptr;
  uint32_t* ws_row = reinterpret_cast<uint32_t*>(t.ws_scores + (int64_t)rl * t.ws_ld);
  const bool keep = !given && t.materialize;
  const RowKeys<T, DI> src(given, keep ? ws_row : nullptr, t, row, p.seq);
  const uint64_t* tops = t.tops + (int64_t)rl * kUnionCapL;
  const int nw = p.W * kSelWaves;
  constexpr int E = kUnionCapL / kSelThreads;
  switch (p.jw) {
    case 1: long_tail<1, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
    case 2: long_tail<2, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
    case 4: long_tail<4, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
    case 8: long_tail<8, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
    case 16: long_tail<16, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
    default: long_tail<32, E>(src, tops, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh); break;
  }
}

// ================================================================ launch

template <typename T, int DI>
static void launch_pool(const PoolArgs& a, int n_seqs, hipStream_t st) {
  constexpr int G = DI / Vec<T>::N;
  const int64_t threads = (int64_t)a.max_new * G;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_seqs);
  hipLaunchKernelGGL((pool_kernel<T, DI>), grid, dim3(256), 0, st, a);
}

template <typename T, int DI, int HI>
static void launch_scores(const IdxArgs& a, int n_rows, int max_n, float* scores, int64_t ld,
                          hipStream_t st) {
  dim3 grid((unsigned)((max_n + kChunk - 1) / kChunk), (unsigned)n_rows);
  hipLaunchKernelGGL((scores_kernel<T, DI, HI>), grid, dim3(256), 0, st, a, scores, ld);
}

template <typename T, int DI, int HI>
static void launch_topk(const TopkArgs& t, int rows, hipStream_t st) {
  dim3 grid((unsigned)t.w_max, (unsigned)rows);
  if (t.ucap == kUnionCapL) {
    hipLaunchKernelGGL((topk_kernel<T, DI, HI, kUnionCapL>), grid, dim3(256), 0, st, t);
    hipLaunchKernelGGL((topk_tail_kernel<T, DI>), dim3((unsigned)rows), dim3(256), 0, st, t);
  } else if (t.ucap == kUnionCapM) {
    hipLaunchKernelGGL((topk_kernel<T, DI, HI, kUnionCapM>), grid, dim3(256), 0, st, t);
  } else {
    hipLaunchKernelGGL((topk_kernel<T, DI, HI, kUnionCap>), grid, dim3(256), 0, st, t);
  }
}

// compile-time indexer head count: the real count rounded up to 2, 4 or 8
// (padding heads carry zero weight and zero query)
template <typename T, int DI, class F>
static void with_hi(int hi, F&& f) {
  if (hi <= 2) f(std::integral_constant<int, 2>{});
  else if (hi <= 4) f(std::integral_constant<int, 4>{});
  else f(std::integral_constant<int, 8>{});
}

template <class F>
static void with_types(int dtype, int di, F&& f) {
  auto go = [&](auto tag) {
    using T = decltype(tag);
    switch (di) {
      case 16: f(T{}, std::integral_constant<int, 16>{}); break;
      case 32: f(T{}, std::integral_constant<int, 32>{}); break;
      case 64: f(T{}, std::integral_constant<int, 64>{}); break;
      case 128: f(T{}, std::integral_constant<int, 128>{}); break;
      default: break;
    }
  };
  if (dtype == QSA_F32) go(float{});
  else go(bf16_t{});
}

void run_pool(const PoolArgs& a, int dtype, int di, int n_seqs, hipStream_t st) {
  with_types(dtype, di, [&](auto tag, auto dic) {
    launch_pool<decltype(tag), decltype(dic)::value>(a, n_seqs, st);
  });
}

void run_pool_rows(const IdxArgs& a, const void* kidx, int dtype, int di, int n_rows,
                   hipStream_t st) {
  with_types(dtype, di, [&](auto tag, auto dic) {
    hipLaunchKernelGGL((pool_rows_kernel<decltype(tag), decltype(dic)::value>),
                       dim3((unsigned)n_rows), dim3(64), 0, st, a, kidx);
  });
}

void run_scores(const IdxArgs& a, int dtype, int di, int n_rows, int max_n, float* scores,
                int64_t ld, hipStream_t st) {
  with_types(dtype, di, [&](auto tag, auto dic) {
    using T = decltype(tag);
    constexpr int DI = decltype(dic)::value;
    with_hi<T, DI>(a.hi, [&](auto hic) {
      launch_scores<T, DI, decltype(hic)::value>(a, n_rows, max_n, scores, ld, st);
    });
  });
}

void run_topk(const TopkArgs& t, int dtype, int di, int rows, hipStream_t st) {
  with_types(dtype, di, [&](auto tag, auto dic) {
    using T = decltype(tag);
    constexpr int DI = decltype(dic)::value;
    with_hi<T, DI>(t.idx.hi, [&](auto hic) {
      launch_topk<T, DI, decltype(hic)::value>(t, rows, st);
    });
  });
}

}  // namespace qsa
