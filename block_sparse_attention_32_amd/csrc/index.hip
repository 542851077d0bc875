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
// G = 16 B / lane-vector lanes cooperate on one row so each load
// instruction reads whole rows, fully coalesced.
#include "index.hpp"
#include "select.hpp"

namespace qsa {

// ================================================================ pooling

template <typename T, int DI>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  constexpr int V = Vec<T>::N;
  constexpr int G = DI / V;  // lanes per block row
  const int s = blockIdx.y;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int bl = gid / G, part = gid % G;
  if (bl >= a.max_new) return;
  const int b0 = a.blk_begin[s];
  const int b = (b0 < 0 ? 0 : b0) + bl;
  const int len = min(a.seq_len[s], a.max_seq_len);
  if (b >= len / kBlock) return;
  const T* kidx = static_cast<const T*>(a.kidx);
  T* kbar = static_cast<T*>(a.kbar);
  const int64_t row0 = a.pm.token_slot(s, b * kBlock);  // 4 rows, one page
  const T* src = kidx + row0 * DI + part * V;
  float r0[V], r1[V], r2[V], r3[V], o[V];
  Vec<T>::load(src, r0);
  Vec<T>::load(src + DI, r1);
  Vec<T>::load(src + 2 * DI, r2);
  Vec<T>::load(src + 3 * DI, r3);
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] = (((r0[i] + r1[i]) + r2[i]) + r3[i]) * 0.25f;
  Vec<T>::store(kbar + a.pm.block_slot(s, b) * DI + part * V, o);
}

// ================================================================ scores

// Per-thread slice of one query row's indexer: this lane's V dims of every
// head, and the head weights.
template <typename T, int DI>
struct IdxQuery {
  static constexpr int V = Vec<T>::N;
  static constexpr int G = DI / V;
  float q[kMaxIdxHeads][V];
  float w[kMaxIdxHeads];
  __device__ __forceinline__ void load(const T* q_idx_row, const float* w_row,
                                       int hi, int part) {
#pragma unroll
    for (int h = 0; h < kMaxIdxHeads; ++h) {
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
  // score of the row whose V-slice this lane loaded into x; all G lanes of
  // the group return the same value
  __device__ __forceinline__ float score(const float (&x)[V]) const {
    float d[kMaxIdxHeads];
#pragma unroll
    for (int h = 0; h < kMaxIdxHeads; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) acc = fmaf(q[h][i], x[i], acc);
      d[h] = acc;
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
#pragma unroll
      for (int h = 0; h < kMaxIdxHeads; ++h) d[h] += __shfl_xor(d[h], off);
    }
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxIdxHeads; ++h) s = fmaf(w[h], fmaxf(d[h], 0.0f), s);
    return canon_zero(s);
  }
};

// Scores of blocks [c0, c0 + kChunk) of one row (blocks >= n get key 0 and
// score 0), computed by the whole workgroup.  keys[i] receives the ordered
// key of block c0 + i; if sc_out is given, sc_out[i] receives the score
// (for i < n - c0).
template <typename T, int DI>
__device__ void chunk_scores(const IdxArgs& a, int seq, int n, int c0,
                             const IdxQuery<T, DI>& iq, uint32_t* keys,
                             float* sc_out) {
  constexpr int V = Vec<T>::N;
  constexpr int G = DI / V;
  constexpr int RPI = 256 / G;           // rows per workgroup iteration
  constexpr int NIT = kChunk / RPI;      // iterations per chunk
  constexpr int U = NIT < 8 ? NIT : 8;   // loads in flight per thread
  const T* kbar = static_cast<const T*>(a.kbar);
  const int gi = threadIdx.x / G, part = threadIdx.x % G;
#pragma unroll 1
  for (int it0 = 0; it0 < NIT; it0 += U) {
    float x[U][V];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = c0 + (it0 + u) * RPI + gi;
      ok[u] = b < n;
      if (ok[u]) {
        Vec<T>::load(kbar + a.pm.block_slot(seq, b) * DI + part * V, x[u]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) x[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (it0 + u) * RPI + gi;
      float s = iq.score(x[u]);
      if (part == 0) keys[i] = ok[u] ? score_key(s) : 0u;
    }
  }
  __syncthreads();
  if (sc_out != nullptr) {
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
      if (c0 + i < n) {
        uint32_t k = keys[i];
        uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
        sc_out[i] = __uint_as_float(u);
      }
    }
  }
}

template <typename T, int DI>
__global__ void __launch_bounds__(256) scores_kernel(IdxArgs a, float* scores,
                                                     int64_t ld) {
  __shared__ uint32_t keys[kChunk];
  const int row = blockIdx.y;
  const int seq = a.seq_of(row);
  const int n = a.pos_of(row) / kBlock;
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= n) return;
  IdxQuery<T, DI> iq;
  iq.load(static_cast<const T*>(a.q_idx) + (int64_t)row * a.hi * DI,
          a.w + (int64_t)row * a.hi, a.hi, threadIdx.x % IdxQuery<T, DI>::G);
  chunk_scores<T, DI>(a, seq, n, c0, iq, keys, scores + (int64_t)row * ld + c0);
}

// ================================================================ top-k

// Per-row plan shared by both passes.
struct RowPlan {
  int seq, n, W, jw, sc;
  __device__ __forceinline__ RowPlan(const TopkArgs& t, int row) {
    seq = t.idx.seq_of(row);
    n = t.idx.pos_of(row) / kBlock;
    W = (n + kChunk - 1) / kChunk;
    jw = row_jw(n, t.top_k);
    sc = W > 0 ? kSlotCap / W : 0;
  }
};

// key of candidate e of a row, from whichever score source is available
template <typename T, int DI>
struct ScoreKey {
  const TopkArgs* t;
  int row_local, row, seq;
  IdxQuery<T, DI>* iq;  // fused recompute (lane-local full dot product)
  const float* src;     // stored scores of this row, or null
  __device__ __forceinline__ uint32_t operator()(int e) const {
    if (src != nullptr) return score_key(src[e]);
    // recompute: this lane alone reads the whole pooled row
    const T* kbar = static_cast<const T*>(t->idx.kbar);
    const T* p = kbar + t->idx.pm.block_slot(seq, e) * DI;
    float d[kMaxIdxHeads];
#pragma unroll
    for (int h = 0; h < kMaxIdxHeads; ++h) d[h] = 0.0f;
    for (int c = 0; c < DI; c += Vec<T>::N) {
      float x[Vec<T>::N];
      Vec<T>::load(p + c, x);
      const T* qrow = static_cast<const T*>(t->idx.q_idx) + (int64_t)row * t->idx.hi * DI;
      for (int h = 0; h < t->idx.hi; ++h) {
#pragma unroll
        for (int i = 0; i < Vec<T>::N; ++i)
          d[h] = fmaf(to_f32(qrow[h * DI + c + i]), x[i], d[h]);
      }
    }
    float s = 0.0f;
    for (int h = 0; h < t->idx.hi; ++h)
      s = fmaf(t->idx.w[(int64_t)row * t->idx.hi + h], fmaxf(d[h], 0.0f), s);
    return score_key(s);
  }
};

struct SelfId {
  __device__ __forceinline__ int32_t operator()(int e) const { return e; }
};

__device__ __forceinline__ void write_all(int32_t* sel_row, int32_t* n_sel, int row,
                                          int n, int top_k) {
  for (int j = threadIdx.x; j < top_k; j += blockDim.x) sel_row[j] = j < n ? j : -1;
  if (threadIdx.x == 0) n_sel[row] = n;
}

// Exact selection over every candidate of a row straight from a score
// source (used for short rows and as the fallback of long rows).
template <class Get>
__device__ void select_full(const Get& get, int n, int top_k, int32_t* sel_row,
                            int32_t* n_sel, int row, SelShared& sh) {
  uint32_t thr;
  int r;
  radix_kth(get, n, top_k, sh, thr, r);
  emit_topk(get, SelfId{}, n, thr, r, sel_row, top_k, sh);
  if (threadIdx.x == 0) n_sel[row] = top_k;
}

struct LdsKeys {
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int e) const { return k[e]; }
};
struct LdsIds {
  const int32_t* id;
  __device__ __forceinline__ int32_t operator()(int e) const { return id[e]; }
};

// Pass A: scores of one chunk of one row; per-wave top-jw keys as the
// chunk's contribution to a lower bound of the row's k-th score.  The last
// chunk of a row either selects directly (short rows, all scores stored)
// or turns the collected keys into the bound tau.
template <typename T, int DI>
__global__ void __launch_bounds__(256) topk_pass_a(TopkArgs t) {
  __shared__ uint32_t keys[kChunk];
  __shared__ uint32_t uni[kUnionCap];
  __shared__ SelShared sh;
  __shared__ uint32_t flag;
  const int rl = blockIdx.y, row = t.row0 + rl, c = blockIdx.x;
  const RowPlan p(t, row);
  int32_t* sel_row = t.sel + (int64_t)row * t.top_k;
  if (p.n <= t.top_k) {
    if (c == 0) write_all(sel_row, t.n_sel, row, p.n, t.top_k);
    return;
  }
  const bool direct = p.n <= kDirectCap;
  const float* given = t.scores ? t.scores + (int64_t)row * t.ld : nullptr;
  if (direct && given) {  // all scores are stored already: one workgroup
    if (c != 0) return;
    for (int e = threadIdx.x; e < p.n; e += blockDim.x) uni[e] = score_key(given[e]);
    __syncthreads();
    select_full(LdsKeys{uni}, p.n, t.top_k, sel_row, t.n_sel, row, sh);
    return;
  }
  if (c >= p.W) return;
  const int c0 = c * kChunk;
  float* ws_row = t.ws_scores ? t.ws_scores + (int64_t)rl * t.ws_ld : nullptr;
  const bool store = ws_row != nullptr && (direct || t.materialize);
  if (given) {
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x)
      keys[i] = (c0 + i < p.n) ? score_key(given[c0 + i]) : 0u;
    __syncthreads();
  } else {
    IdxQuery<T, DI> iq;
    iq.load(static_cast<const T*>(t.idx.q_idx) + (int64_t)row * t.idx.hi * DI,
            t.idx.w + (int64_t)row * t.idx.hi, t.idx.hi,
            threadIdx.x % IdxQuery<T, DI>::G);
    chunk_scores<T, DI>(t.idx, p.seq, p.n, c0, iq, keys, store ? ws_row + c0 : nullptr);
  }
  if (!direct) {
    // per-wave top-jw keys of this chunk (key 0 = none left)
    const int wave = threadIdx.x / kWave, lane = lane_id();
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = keys[wave * 256 + lane + 64 * i];
    uint32_t* dst = t.tops + (int64_t)rl * kUnionCap + (c * kSelWaves + wave) * p.jw;
    for (int j = 0; j < p.jw; ++j) {
      uint32_t lm = max(max(v[0], v[1]), max(v[2], v[3]));
      uint32_t wm = wave_max_u32(lm);
      uint64_t b = ballot(lm == wm);
      if (lane == (int)(__ffsll((unsigned long long)b) - 1)) {
        bool done = false;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!done && v[i] == wm) { v[i] = 0u; done = true; }
      }
      if (lane == 0) dst[j] = wm;
    }
  }
  if (!arrive_last(t.cnt_a + rl, (uint32_t)p.W, &flag)) return;
  if (direct) {
    for (int e = threadIdx.x; e < p.n; e += blockDim.x)
      uni[e] = score_key(__builtin_nontemporal_load(ws_row + e));
    __syncthreads();
    select_full(LdsKeys{uni}, p.n, t.top_k, sel_row, t.n_sel, row, sh);
    return;
  }
  const int un = p.W * kSelWaves * p.jw;
  const uint32_t* src = t.tops + (int64_t)rl * kUnionCap;
  for (int e = threadIdx.x; e < un; e += blockDim.x) uni[e] = __builtin_nontemporal_load(src + e);
  __syncthreads();
  uint32_t tau = 0u;
  if (un >= t.top_k) {
    int r;
    radix_kth(LdsKeys{uni}, un, t.top_k, sh, tau, r);
  }
  if (threadIdx.x == 0) t.tau[rl] = tau;
}

// Pass B: the survivors (key >= tau) of one chunk, in index order, into the
// chunk's slots; the last chunk of a row gathers all survivors in order and
// selects the k best exactly.
template <typename T, int DI>
__global__ void __launch_bounds__(256) topk_pass_b(TopkArgs t) {
  __shared__ uint32_t keys[kChunk];
  __shared__ uint32_t ckey[kSelCap];
  __shared__ int32_t cid[kSelCap];
  __shared__ SelShared sh;
  __shared__ uint32_t flag;
  const int rl = blockIdx.y, row = t.row0 + rl, c = blockIdx.x;
  const RowPlan p(t, row);
  if (p.n <= kDirectCap || c >= p.W) return;
  int32_t* sel_row = t.sel + (int64_t)row * t.top_k;
  const int c0 = c * kChunk;
  const float* given = t.scores ? t.scores + (int64_t)row * t.ld : nullptr;
  const float* stored = given ? given
                              : (t.materialize ? t.ws_scores + (int64_t)rl * t.ws_ld : nullptr);
  if (stored) {
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x)
      keys[i] = (c0 + i < p.n) ? score_key(stored[c0 + i]) : 0u;
    __syncthreads();
  } else {
    IdxQuery<T, DI> iq;
    iq.load(static_cast<const T*>(t.idx.q_idx) + (int64_t)row * t.idx.hi * DI,
            t.idx.w + (int64_t)row * t.idx.hi, t.idx.hi,
            threadIdx.x % IdxQuery<T, DI>::G);
    chunk_scores<T, DI>(t.idx, p.seq, p.n, c0, iq, keys, nullptr);
  }
  const uint32_t tau = t.tau[rl];
  // keys 0 are padding past n; a real key is always > 0
  const int wave = threadIdx.x / kWave, lane = lane_id();
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t k = keys[wave * 256 + i * 64 + lane];
    cnt += __popcll(ballot(k != 0u && k >= tau));
  }
  if (lane == 0) sh.wcnt[0][wave] = cnt;
  __syncthreads();
  uint32_t base = 0, total = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    base += (w < wave) ? sh.wcnt[0][w] : 0u;
    total += sh.wcnt[0][w];
  }
  uint2* slot = t.slots + (int64_t)rl * kSlotCap + (int64_t)c * p.sc;
  if (total <= (uint32_t)p.sc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int li = wave * 256 + i * 64 + lane;
      uint32_t k = keys[li];
      bool take = k != 0u && k >= tau;
      uint64_t m = ballot(take);
      if (take) slot[base + lanes_below(m)] = make_uint2(k, (uint32_t)(c0 + li));
      base += __popcll(m);
    }
  } else if (threadIdx.x == 0) {
    atomicOr(t.flags + rl, 1u);
  }
  if (threadIdx.x == 0) t.chunk_cnt[(int64_t)rl * t.w_max + c] = total;
  if (!arrive_last(t.cnt_b + rl, (uint32_t)p.W, &flag)) return;

  // ---- last chunk of the row: gather survivors in index order
  bool overflow = __builtin_nontemporal_load(t.flags + rl) != 0u;
  uint32_t m_total = 0;
  if (!overflow) {
    // thread th owns chunks [th*q, th*q+q)
    const int q = (p.W + kSelThreads - 1) / kSelThreads;
    uint32_t mine = 0;
    const uint32_t* cc = t.chunk_cnt + (int64_t)rl * t.w_max;
    for (int j = 0; j < q; ++j) {
      int ch = threadIdx.x * q + j;
      if (ch < p.W) mine += __builtin_nontemporal_load(cc + ch);
    }
    uint32_t off = block_excl_scan(mine, sh, m_total);
    if (m_total <= (uint32_t)kSelCap) {
      for (int j = 0; j < q; ++j) {
        int ch = threadIdx.x * q + j;
        if (ch >= p.W) break;
        uint32_t nc = __builtin_nontemporal_load(cc + ch);
        const uint2* sl = t.slots + (int64_t)rl * kSlotCap + (int64_t)ch * p.sc;
        for (uint32_t i = 0; i < nc; ++i) {
          const uint2 v = sl[i];
          ckey[off + i] = v.x;
          cid[off + i] = (int32_t)v.y;
        }
        off += nc;
      }
    } else {
      overflow = true;
    }
    __syncthreads();
  }
  if (!overflow) {
    uint32_t thr;
    int r;
    radix_kth(LdsKeys{ckey}, (int)m_total, t.top_k, sh, thr, r);
    emit_topk(LdsKeys{ckey}, LdsIds{cid}, (int)m_total, thr, r, sel_row, t.top_k, sh);
    if (threadIdx.x == 0) t.n_sel[row] = t.top_k;
  } else {
    // rare: more survivors than the slots hold (heavy ties); exact select
    // over every candidate, recomputing scores if none are stored
    IdxQuery<T, DI> dummy;
    ScoreKey<T, DI> get{&t, rl, row, p.seq, &dummy, stored};
    select_full(get, p.n, t.top_k, sel_row, t.n_sel, row, sh);
  }
  if (threadIdx.x == 0) t.flags[rl] = 0u;
}

// ================================================================ launch

template <typename T, int DI>
static void launch_pool(const PoolArgs& a, int n_seqs, hipStream_t st) {
  constexpr int G = DI / Vec<T>::N;
  int64_t threads = (int64_t)a.max_new * G;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_seqs);
  hipLaunchKernelGGL((pool_kernel<T, DI>), grid, dim3(256), 0, st, a);
}

template <typename T, int DI>
static void launch_scores(const IdxArgs& a, int n_rows, int max_n, float* scores,
                          int64_t ld, hipStream_t st) {
  dim3 grid((unsigned)((max_n + kChunk - 1) / kChunk), (unsigned)n_rows);
  hipLaunchKernelGGL((scores_kernel<T, DI>), grid, dim3(256), 0, st, a, scores, ld);
}

template <typename T, int DI>
static void launch_topk(const TopkArgs& t, int rows, hipStream_t st) {
  dim3 grid((unsigned)t.w_max, (unsigned)rows);
  hipLaunchKernelGGL((topk_pass_a<T, DI>), grid, dim3(256), 0, st, t);
  hipLaunchKernelGGL((topk_pass_b<T, DI>), grid, dim3(256), 0, st, t);
}

#define QSA_DISPATCH_DI(T, DI, CALL)                  \
  switch (DI) {                                       \
    case 16: { constexpr int kDi = 16; CALL; } break; \
    case 32: { constexpr int kDi = 32; CALL; } break; \
    case 64: { constexpr int kDi = 64; CALL; } break; \
    case 128: { constexpr int kDi = 128; CALL; } break; \
    default: break;                                   \
  }

void run_pool(const PoolArgs& a, int dtype, int di, int n_seqs, hipStream_t st) {
  if (dtype == QSA_F32) { QSA_DISPATCH_DI(float, di, (launch_pool<float, kDi>(a, n_seqs, st))); }
  else { QSA_DISPATCH_DI(bf16_t, di, (launch_pool<bf16_t, kDi>(a, n_seqs, st))); }
}

void run_scores(const IdxArgs& a, int dtype, int di, int n_rows, int max_n, float* scores,
                int64_t ld, hipStream_t st) {
  if (dtype == QSA_F32) {
    QSA_DISPATCH_DI(float, di, (launch_scores<float, kDi>(a, n_rows, max_n, scores, ld, st)));
  } else {
    QSA_DISPATCH_DI(bf16_t, di, (launch_scores<bf16_t, kDi>(a, n_rows, max_n, scores, ld, st)));
  }
}

void run_topk(const TopkArgs& t, int dtype, int di, int rows, hipStream_t st) {
  if (dtype == QSA_F32) { QSA_DISPATCH_DI(float, di, (launch_topk<float, kDi>(t, rows, st))); }
  else { QSA_DISPATCH_DI(bf16_t, di, (launch_topk<bf16_t, kDi>(t, rows, st))); }
}

}  // namespace qsa
