// Argument blocks and host entry points of the indexer kernels.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace qsa {

constexpr int kChunk = 1024;        // candidate blocks per workgroup (4 per thread)
constexpr int kChunkWaves = 4;      // waves of a top-k workgroup (one run of 256 candidates each)
constexpr int kDirectCap = 8192;    // rows with <= this many candidates select in one pass
constexpr int kUnionCap = 4096;     // (key, id) pairs of the per-wave tops of one row
constexpr int kLargeTopk = 512;     // larger selections use the wider unions below
constexpr int kUnionCapM = 8192;    // larger selections, rows of up to kUnionMChunks chunks
constexpr int kUnionCapL = 16384;   // larger selections, longer rows (tail in its own kernel)
constexpr int kUnionMChunks = 256;
constexpr int kSelCap = 4096;       // survivors gathered into LDS for the final select
constexpr int kMaxIdxHeads = 8;
constexpr int kMaxJw = 16;
constexpr int kMaxJwL = 32;         // per-wave tops of a large selection
constexpr int kArriveGroup = 32;    // chunks per first-level arrival counter of a row
constexpr int kCtrStride = 64;      // words between arrival counters (one 256-byte line each)

// Arrival counters of one row of the top-k: one, or with more than
// kArriveGroup chunks a top counter and one per group of kArriveGroup.
__host__ __device__ inline int arrive_slots(int w_max) {
  return w_max > kArriveGroup ? 1 + (w_max + kArriveGroup - 1) / kArriveGroup : 1;
}

// Per-wave top count: each wave of each chunk publishes its jw best
// (key, id) pairs: the largest power of two that fits the call's union
// capacity ucap, at most kMaxJw (kMaxJwL for the wider unions).  The union
// is kUnionCap for selections of at most kLargeTopk blocks; larger ones
// take kUnionCapM, or kUnionCapL when the longest row has more than
// kUnionMChunks chunks.  Rows that take this path have at least 9 chunks
// (more than kDirectCap candidates); the union then holds 4 * W * jw >= 576
// pairs (1152 for the wider unions), at least half its capacity from
// ucap / 64 chunks on.  A union smaller than top_k gives no bound: such rows
// select exactly over every key.  A larger jw makes a wave whose jw-th key
// still reaches the bound (a "saturated" wave, rescanned in full) rarer.
__host__ __device__ inline int union_cap(int top_k, int w_max) {
  if (top_k <= kLargeTopk) return kUnionCap;
  return w_max <= kUnionMChunks ? kUnionCapM : kUnionCapL;
}
__host__ __device__ inline int row_jw(int n, int ucap) {
  int W = (n + kChunk - 1) / kChunk;
  if (W <= 0) return 1;
  const int cap = ucap / (4 * W);
  const int jmax = ucap == kUnionCap ? kMaxJw : kMaxJwL;
  int jw = 1;
  while (jw * 2 <= cap && jw * 2 <= jmax) jw *= 2;  // a power of two
  return jw;
}

struct PoolArgs {
  PageMap pm;
  const void* kidx;
  void* kbar;
  const int32_t* seq_len;
  const int32_t* blk_begin;
  int max_new;
  int max_seq_len;       // seq_len is clamped to it
};

struct IdxArgs {
  PageMap pm;
  const void* kbar;
  const void* q_idx;     // [T][hi][Di]
  const float* w;        // [T][hi]
  int hi;
  const int32_t* seq_id;
  const int32_t* pos;
  int n_seqs;            // seq_id is clamped to [0, n_seqs)
  int max_pos;           // pos is clamped to [0, max_pos]
  __device__ __forceinline__ int seq_of(int row) const {
    return clamp_flag(seq_id[row], 0, n_seqs - 1, QSA_DEBUG_BAD_ROW);
  }
  __device__ __forceinline__ int pos_of(int row) const {
    return clamp_flag(pos[row], 0, max_pos, QSA_DEBUG_BAD_ROW);
  }
};

struct TopkArgs {
  IdxArgs idx;
  const float* scores;   // caller's scores or null (fused)
  int64_t ld;
  int row0;              // first row of this batch
  int top_k;
  int32_t* sel;
  int32_t* n_sel;
  int w_max;             // chunks of the longest row
  float* ws_scores;      // [R][ws_ld] keys of rows of at most kDirectCap candidates
  int64_t ws_ld;
  uint32_t* cnt;         // [R][ctr_slots][kCtrStride] arrival counters (arrive_slots)
  int ctr_slots;
  int ucap;              // union capacity per row (union_cap)
  uint64_t* tops;        // [R][ucap] (block id << 32 | key)
  uint32_t* nxt;         // [R][w_max * 4] largest key of each wave not in its tops (0: none)
  const void* pool_kidx; // non-null: pool each row's newest complete block first
};

// ---- MFMA prefill indexer (index_mfma.hip)
constexpr int kPQT = 128;         // query rows per workgroup tile (8 waves x 16)
constexpr int kPThreads = 512;    // threads of a scoring workgroup
constexpr int kPGrp = 256;        // pooled keys staged per group
constexpr int kPUnion = 4096;     // union entries (group maxima) per row
constexpr int kPSurvCap = 8192;   // survivor slots per row, over all splits
constexpr int kPSelCap = 8192;    // survivors a row's exact select stages in LDS
constexpr int kPMaxStride = 8;    // largest group sampling stride of P1
constexpr int kPMaxSplits = 16;   // block splits per tile
constexpr int kPMinRows = 64;     // fused top-k of at least this many rows uses it
constexpr int kPRowBatch = 32768; // rows per launch
constexpr int kPWave = 16;        // survivors per lane of the one-wave select (1,024 per row)

struct PIdxArgs {
  IdxArgs idx;
  int row0, rows, top_k;
  int splits;                // block splits per query tile
  uint32_t* uni;             // [rows][kPUnion] group maxima (P1)
  uint32_t* tau;             // [rows] lower bound of the k-th key (P2)
  int32_t* tile_stride;      // [tiles] sampling stride of P1
  int32_t* row_stride;       // [rows] stride used for each row's union
  uint64_t* surv;            // [rows][splits][kPSurvCap / splits] (block << 32 | score bits)
  uint32_t* surv_cnt;        // [rows][splits]
  uint32_t* done;            // [rows] set by the one-wave select, cleared by the fallback
  uint32_t* fb_cnt;          // [2] rows listed for the exact fallback; its arrival counter
  int32_t* fb_list;          // [rows] those rows (batch-local index)
  int32_t* sel;
  int32_t* n_sel;
};
constexpr int kPFallbackWgs = 64;  // workgroups of the fallback kernel (they loop over its list)

bool pidx_supported(int dtype, int di, int hi);
void run_pidx(const PIdxArgs& a, int di, hipStream_t st);

void run_pool(const PoolArgs& a, int dtype, int di, int n_seqs, hipStream_t st);
void run_scores(const IdxArgs& a, int dtype, int di, int n_rows, int max_n, float* scores,
                int64_t ld, hipStream_t st);
void run_topk(const TopkArgs& t, int dtype, int di, int rows, hipStream_t st);
// block pos/B - 1 of every row's sequence (rows with pos >= B), pooled
void run_pool_rows(const IdxArgs& a, const void* kidx, int dtype, int di, int n_rows,
                   hipStream_t st);

}  // namespace qsa
