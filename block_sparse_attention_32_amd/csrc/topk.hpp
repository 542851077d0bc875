// Exact per-query top-k block selection for few rows (decode): the chunked
// top-k kernels.  Instantiated per (element type, indexer dimension) in the
// topk_*.hip translation units, which the library build compiles in
// parallel.
#pragma once

#include "index_device.hpp"
#include "select.hpp"

namespace qsa {

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
struct ScoreKeys {  // keys of caller scores
  const float* s;
  __device__ __forceinline__ uint32_t operator()(int e) const { return score_key(s[e]); }
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
  int64_t n_pages;       // pages in the pool
  int hi, bsh;           // heads; log2(blocks per page)
  // (56 bytes: small enough to travel in registers to the out-of-line
  // selection routines)
  __device__ __forceinline__ RowKeys(const float* g, const uint32_t* st, const TopkArgs& t, int row,
                                     int sq)
      : given(g), stored(st), kbar(static_cast<const T*>(t.idx.kbar)),
        qrow(static_cast<const T*>(t.idx.q_idx) + (int64_t)row * t.idx.hi * DI),
        wrow(t.idx.w + (int64_t)row * t.idx.hi),
        pages(t.idx.pm.table + (int64_t)sq * t.idx.pm.max_pages), n_pages(t.idx.pm.n_pages),
        hi(t.idx.hi),
        bsh(t.idx.pm.bpp_shift()) {}
  __device__ __forceinline__ uint32_t operator()(int e) const {
    if (given != nullptr) return score_key(given[e]);
    if (stored != nullptr) return stored[e];
    const int64_t slot =
        ((int64_t)checked_page(pages[e >> bsh], n_pages) << bsh) + (e & ((1 << bsh) - 1));
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

// Keys of run r of a long row (candidates [kRun r, kRun r + kRun), one
// scoring wave's), produced by the calling wave into dst[0, kRun): from the
// caller's scores, or recomputed with the scoring pass's own vector path
// (run_scores), which gives the keys the tops were taken from, bit for bit.
template <typename T, int DI, int HI>
struct RunKeys {
  const IdxArgs& idx;
  const float* given;
  const typename RowQuery<T, DI, HI>::type& iq;
  int seq, n;
  __device__ __forceinline__ void operator()(int r, uint32_t* dst) const {
    const int b0 = r * kRun;
    if (given != nullptr) {
      const int lane = lane_id();
#pragma unroll
      for (int j = 0; j < kRun / kWave; ++j) {
        const int e = b0 + kWave * j + lane;
        dst[kWave * j + lane] = e < n ? score_key(given[e]) : 0u;
      }
    } else {
      run_scores<T, DI, HI>(idx, seq, n, b0, iq, dst);
    }
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
// (key, id) pairs, and the largest of its other keys.  The last chunk takes
// tau = the k-th largest key of all published pairs: tau is a key of the
// row, and at least k keys are >= tau, so tau never exceeds the row's k-th
// largest key and every selected block has key >= tau.  A wave whose
// largest unpublished key is below tau has all of its keys >= tau among its
// published pairs; only a wave whose unpublished key reaches tau
// ("saturated": at least jw + 1 of its keys reach tau, rare) is rescanned.  The survivors are gathered
// wave by wave, ascending ids inside each wave, so they come out in
// ascending id order, and the exact radix select + ordered emission of
// select.hpp picks the k best with ties to the lower id.
static_assert(kChunkWaves == kSelWaves, "a top-k workgroup's waves are its runs");
static_assert(kChunk == kSelWaves * kRun, "a chunk is four runs; its keys[] holds four rescored runs");
constexpr int kMaxSat = 64;  // saturated waves rescanned per row (else exact fallback)
constexpr int kWaveSel = 16;  // survivors per lane of the one-wave final select (1,024)

// LDS of the tail of a long row.
struct LongShared {
  alignas(16) uint32_t skey[kSelCap];  // survivors, in ascending id order
  int32_t sid[kSelCap];
  int32_t sat_w[kMaxSat];  // saturated runs
  uint32_t sat_cnt[kMaxSat], sat_off[kMaxSat];
  uint32_t n_sat;
  // skey and sid back to back: the staging area of the coalesced reads
  // (stage_chunks) before any survivor is placed
  __device__ __forceinline__ uint4* stage() { return reinterpret_cast<uint4*>(skey); }
};
static_assert(offsetof(LongShared, sid) == sizeof(uint32_t) * kSelCap &&
                  2 * sizeof(uint32_t) * kSelCap == 16 * kStageChunks * kSelThreads,
              "skey and sid together are one 32 KB staging area");

// Keys of elements 4c .. 4c + 3 of a row of n >= 1 (0 past n), read with
// no branch, so that a thread's loads are all in flight together: every
// read is clamped into the row and the elements past n are then zeroed.
__device__ __forceinline__ uint4 mask_chunk(uint4 v, int c, int n) {
  const int e = 4 * c;
  return uint4{e < n ? v.x : 0u, e + 1 < n ? v.y : 0u, e + 2 < n ? v.z : 0u,
               e + 3 < n ? v.w : 0u};
}
template <class Get>
__device__ __forceinline__ uint4 key_chunk(const Get& get, int c, int n) {
  const int e = 4 * c;
  return mask_chunk(uint4{get(min(e, n - 1)), get(min(e + 1, n - 1)), get(min(e + 2, n - 1)),
                          get(min(e + 3, n - 1))},
                    c, n);
}
// Stored keys: the workspace row is 16-byte aligned and holds a multiple of
// four keys, at least n, so the chunk holding element n - 1 is whole.
struct StoredKeys {
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int e) const { return k[e]; }
};
__device__ __forceinline__ uint4 key_chunk(const StoredKeys& get, int c, int n) {
  const uint4 v = *reinterpret_cast<const uint4*>(get.k + 4 * min(c, (n - 1) >> 2));
  return mask_chunk(v, c, n);
}

// Tail of a long row (the last chunk to finish), JW keys per published run.
// Thread t holds union entries [E t, E t + E) -- whole runs, E = union cap /
// 256 -- in registers, loaded at once, with the largest unpublished key of
// each of its runs (nxt).  tau = the k-th largest union key (low bits past
// two radix digits cleared); a run whose unpublished key reaches tau is
// saturated and rescanned: wave w rescores runs w, w + 4, ... into its
// quarter of rk (kRun keys each) with run_keys, counts them, and -- when
// there are at most four, so that each stays in LDS -- places them from
// there (else it rescores them).  The other runs' survivors (key >= tau)
// are placed in id order straight from the registers, each run's entries
// ranked by id (a run lists one wave's keys best first).  Then the exact
// select among the survivors; src (every key of the row) serves the rare
// select over all keys.
template <int JW, int E, class Src, class Run>
__device__ __forceinline__ void long_tail(const Src& src, const Run& run_keys, uint32_t* rk,
                                          const uint64_t* tops, const uint32_t* nxt, int nw,
                                          int n, int top_k, int32_t* sel_row, int32_t* n_sel,
                                          int row, LongShared& ls, SelShared& sh) {
  static_assert(JW <= E, "a thread holds whole runs");
  constexpr int R = E / JW;
  const int un = nw * JW;
  const int e0 = (int)threadIdx.x * E;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  uint32_t k[E];
  int32_t id[E];
  uint32_t nx[R];  // largest unpublished key of each of this thread's runs
  if constexpr (E == 2 * kStageChunks) {
    // the 4,096-pair union: read coalesced, through LDS, every chunk of the
    // row's 4,096 entries with no branch (pairs past un are then zeroed)
    uint4 ch[kStageChunks];
    stage_chunks(
        [&](int c) -> uint4 {
          const uint4 v = *reinterpret_cast<const uint4*>(tops + 2 * c);
          const bool lo = 2 * c < un, hi = 2 * c + 1 < un;
          return uint4{lo ? v.x : 0u, lo ? v.y : 0u, hi ? v.z : 0u, hi ? v.w : 0u};
        },
        ls.stage(), ch);
#pragma unroll
    for (int i = 0; i < kStageChunks; ++i) {
      k[2 * i] = ch[i].x;
      id[2 * i] = (int32_t)ch[i].y;
      k[2 * i + 1] = ch[i].z;
      id[2 * i + 1] = (int32_t)ch[i].w;
    }
    bool nx_done = false;
    if constexpr (R == 4) {
      if (e0 + E <= un) {  // the thread's 4 words, 16-byte aligned
        const uint4 n4 = *reinterpret_cast<const uint4*>(nxt + e0 / JW);
        nx[0] = n4.x;
        nx[1] = n4.y;
        nx[2] = n4.z;
        nx[3] = n4.w;
        nx_done = true;
      }
    }
    if (!nx_done) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) nx[rr] = e0 + rr * JW < un ? nxt[e0 / JW + rr] : 0u;
    }
  } else {
    uint64_t v[E];
    if (e0 + E <= un) {
      // whole runs in range (every thread of a full union): 16-byte loads,
      // no per-entry tests (tops rows and the thread's E entries are 16-byte
      // aligned, and so are the thread's R nxt words when R is 4)
      typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));
      const u64x2_t* tp = reinterpret_cast<const u64x2_t*>(tops + e0);
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const u64x2_t t2 = tp[i];
        v[2 * i] = t2.x;
        v[2 * i + 1] = t2.y;
      }
      if constexpr (R == 4) {
        const uint4 n4 = *reinterpret_cast<const uint4*>(nxt + e0 / JW);
        nx[0] = n4.x;
        nx[1] = n4.y;
        nx[2] = n4.z;
        nx[3] = n4.w;
      } else {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) nx[rr] = nxt[e0 / JW + rr];
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = e0 + i < un ? tops[e0 + i] : 0ull;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) nx[rr] = e0 + rr * JW < un ? nxt[e0 / JW + rr] : 0u;
    }
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
    if (e0 + rr * JW < un && nx[rr] >= tau && nx[rr] != 0u) {
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
  const bool runs_kept = ns <= kSelWaves;  // each wave's one run stays in rk
  uint32_t* my_rk = rk + wave * kRun;
  // survivor counts of saturated runs (wave w counts runs w, w + 4, ...,
  // with no workgroup barrier per run)
#pragma unroll 1
  for (int i = wave; fits && i < ns; i += kSelWaves) {
    const int e0 = ls.sat_w[i] * kRun + lane;
    run_keys(ls.sat_w[i], my_rk);
    uint32_t cw = 0;
#pragma unroll
    for (int j = 0; j < kRun / kWave; ++j) {
      const int e = e0 + kWave * j;
      cw += (uint32_t)__popcll(ballot(e < n && my_rk[kWave * j + lane] >= tau));
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
    const int e0 = ls.sat_w[i] * kRun + lane;
    if (!runs_kept) run_keys(ls.sat_w[i], my_rk);
    uint32_t base = ls.sat_off[i];
#pragma unroll
    for (int j = 0; j < kRun / kWave; ++j) {
      const int e = e0 + kWave * j;
      const uint32_t kk = e < n ? my_rk[kWave * j + lane] : 0u;
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
// returns: up to 1,024 candidates go to one wave's bit-by-bit select;
// otherwise thread t holds keys t * EPT .. t * EPT + EPT - 1 in registers
// (read coalesced through the 32 KB LDS area stage), then a register radix
// select and ordered emission.  Kept out of line: it runs once per row.
template <class Get>
__device__ __noinline__ void select_direct(Get get, int n, int top_k, int32_t* sel_row,
                                           int32_t* n_sel, int row, uint4* stage, SelShared& sh) {
  if (n <= kWave * kWaveSel) {
    // few candidates: one wave selects them, bit by bit without barriers
    // (element jj at lane jj % 64, in id order)
    if (threadIdx.x < kWave) {
      const int lane = lane_id();
      uint32_t key[kWaveSel];
      int32_t id[kWaveSel];
#pragma unroll
      for (int i = 0; i < kWaveSel; ++i) {
        const int jj = i * kWave + lane;
        key[i] = jj < n ? get(jj) : 0u;
        id[i] = jj;
      }
      wave_topk_ordered<kWaveSel>(key, id, top_k, sel_row);
      if (lane == 0) n_sel[row] = top_k;
    }
    return;
  }
  constexpr int EPT = kDirectCap / kSelThreads;
  static_assert(EPT == 4 * kStageChunks, "a thread's keys are its staged chunks");
  const int base = (int)threadIdx.x * EPT;
  uint32_t key[EPT];
  int32_t id[EPT];
  {
    uint4 ch[kStageChunks];
    stage_chunks([&](int c) { return key_chunk(get, c, n); }, stage, ch);
#pragma unroll
    for (int i = 0; i < kStageChunks; ++i) {
      key[4 * i] = ch[i].x;
      key[4 * i + 1] = ch[i].y;
      key[4 * i + 2] = ch[i].z;
      key[4 * i + 3] = ch[i].w;
    }
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) id[i] = base + i;
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
    select_direct(ScoreKeys{given}, p.n, t.top_k, sel_row, t.n_sel, row, ls.stage(), sh);
    return;
  }
  if (c >= p.W) return;
  const int c0 = c * kChunk;
  uint32_t* ws_row = reinterpret_cast<uint32_t*>(t.ws_scores + (int64_t)rl * t.ws_ld);
  const bool keep = !given && direct;  // long rows publish tops only
  typename RowQuery<T, DI, HI>::type iq;  // (also rescores saturated runs in the tail)
  if (given) {
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x)
      keys[i] = (c0 + i < p.n) ? score_key(given[c0 + i]) : 0u;
    __syncthreads();
  } else {
    load_row_query<T, DI, HI>(iq, t.idx, row);
    chunk_scores<T, DI, HI>(t.idx, p.seq, p.n, c0, iq, pages, keys);
    if (p.W == 1) {
      // the row's only chunk: every key is in this workgroup's LDS
      // (chunk_scores ends with a barrier), so it selects at once, with no
      // hand-off through memory and no arrival
      select_direct(KeyArray{keys}, p.n, t.top_k, sel_row, t.n_sel, row, ls.stage(), sh);
      return;
    }
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
    // the largest key left: a bound of every unpublished key of the wave
    const uint32_t rest = wave_max_u32(max(max(v[0], v[1]), max(v[2], v[3])));
    if (lane == 0)
      st_agent(t.nxt + (int64_t)rl * t.w_max * kSelWaves + c * kSelWaves + wave, rest);
  }
  if (!OWN_TAIL && !direct) return;  // the tail follows in topk_tail_kernel
  if (!arrive_last_tree<kArriveGroup>(t.cnt + (int64_t)rl * t.ctr_slots * kCtrStride, kCtrStride,
                                      (uint32_t)c, (uint32_t)p.W, &flag))
    return;
  if (direct) {
    select_direct(StoredKeys{ws_row}, p.n, t.top_k, sel_row, t.n_sel, row, ls.stage(), sh);
    return;
  }

  // ---- last chunk of a long row (its scoring LDS, keys[], holds the
  // rescored saturated runs)
  if constexpr (OWN_TAIL) {
    const RowKeys<T, DI> src(given, keep ? ws_row : nullptr, t, row, p.seq);
    const RunKeys<T, DI, HI> rs{t.idx, given, iq, p.seq, p.n};
    const int nw = p.W * kSelWaves;
    constexpr int E = UCAP / kSelThreads;
    const uint32_t* nxt = t.nxt + (int64_t)rl * t.w_max * kSelWaves;
#define QSA_LONG_TAIL(J) \
  long_tail<J, E>(src, rs, keys, tops, nxt, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh)
    switch (p.jw) {
      case 1: QSA_LONG_TAIL(1); break;
      case 2: QSA_LONG_TAIL(2); break;
      case 4: QSA_LONG_TAIL(4); break;
      case 8: QSA_LONG_TAIL(8); break;
      case 16: QSA_LONG_TAIL(16); break;
      default:
        if constexpr (E >= 32) QSA_LONG_TAIL(32);
        break;
    }
#undef QSA_LONG_TAIL
  }
}

// The tail of the long rows of a large selection, after topk_kernel has
// published every chunk's per-wave tops: one workgroup per row.
template <typename T, int DI, int HI>
__global__ void __launch_bounds__(256) topk_tail_kernel(TopkArgs t) {
  __shared__ LongShared ls;
  __shared__ SelShared sh;
  __shared__ uint32_t rk[kSelWaves * kRun];
  const int rl = blockIdx.x, row = t.row0 + rl;
  const RowPlan p(t, row);
  if (p.n <= t.top_k || p.n <= kDirectCap) return;  // done by topk_kernel
  int32_t* sel_row = t.sel + (int64_t)row * t.top_k;
  const float* given = t.scores ? t.scores + (int64_t)row * t.ld : nullptr;
  typename RowQuery<T, DI, HI>::type iq;
  if (!given) load_row_query<T, DI, HI>(iq, t.idx, row);
  const RowKeys<T, DI> src(given, nullptr, t, row, p.seq);
  const RunKeys<T, DI, HI> rs{t.idx, given, iq, p.seq, p.n};
  const uint64_t* tops = t.tops + (int64_t)rl * kUnionCapL;
  const uint32_t* nxt = t.nxt + (int64_t)rl * t.w_max * kSelWaves;
  const int nw = p.W * kSelWaves;
  constexpr int E = kUnionCapL / kSelThreads;
#define QSA_LONG_TAIL_L(J) \
  long_tail<J, E>(src, rs, rk, tops, nxt, nw, p.n, t.top_k, sel_row, t.n_sel, row, ls, sh)
  switch (p.jw) {
    case 1: QSA_LONG_TAIL_L(1); break;
    case 2: QSA_LONG_TAIL_L(2); break;
    case 4: QSA_LONG_TAIL_L(4); break;
    case 8: QSA_LONG_TAIL_L(8); break;
    case 16: QSA_LONG_TAIL_L(16); break;
    default: QSA_LONG_TAIL_L(32); break;
  }
#undef QSA_LONG_TAIL_L
}

// Launches the top-k kernels of one row batch for element type T and
// indexer dimension DI; the compile-time head count is the real count
// rounded up to 2, 4 or 8 (padding heads carry zero weight).
template <typename T, int DI, int HI>
static void launch_topk(const TopkArgs& t, int rows, hipStream_t st) {
  dim3 grid((unsigned)t.w_max, (unsigned)rows);
  if (t.ucap == kUnionCapL) {
    hipLaunchKernelGGL((topk_kernel<T, DI, HI, kUnionCapL>), grid, dim3(256), 0, st, t);
    hipLaunchKernelGGL((topk_tail_kernel<T, DI, HI>), dim3((unsigned)rows), dim3(256), 0, st, t);
  } else if (t.ucap == kUnionCapM) {
    hipLaunchKernelGGL((topk_kernel<T, DI, HI, kUnionCapM>), grid, dim3(256), 0, st, t);
  } else {
    hipLaunchKernelGGL((topk_kernel<T, DI, HI, kUnionCap>), grid, dim3(256), 0, st, t);
  }
}

template <typename T, int DI>
void launch_topk_typed(const TopkArgs& t, int rows, hipStream_t st) {
  if (t.idx.hi <= 2) launch_topk<T, DI, 2>(t, rows, st);
  else if (t.idx.hi <= 4) launch_topk<T, DI, 4>(t, rows, st);
  else launch_topk<T, DI, 8>(t, rows, st);
}

}  // namespace qsa
