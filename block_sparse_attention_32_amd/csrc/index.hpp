// Argument blocks and host entry points of the indexer kernels.
#pragma once

#include "common.hpp"

namespace qsa {

constexpr int kChunk = 1024;        // candidate blocks per workgroup (4 per thread)
constexpr int kDirectCap = 8192;    // rows with <= this many candidates select in one pass
constexpr int kUnionCap = 8192;     // keys of the per-chunk tops of one row
constexpr int kSelCap = 8192;       // survivors gathered into LDS for the final select
constexpr int kSlotCap = 16384;     // survivor slots per row, split evenly over its chunks
constexpr int kMaxIdxHeads = 8;

// per-wave top count of the chunk tops: the union over a row's chunks holds
// about 2k keys, and never more than kUnionCap
__host__ __device__ inline int row_jw(int n, int top_k) {
  int W = (n + kChunk - 1) / kChunk;
  if (W <= 0) return 1;
  int jw = (2 * top_k + 4 * W - 1) / (4 * W);
  jw = jw < 1 ? 1 : (jw > 16 ? 16 : jw);
  while (jw > 1 && 4 * W * jw > kUnionCap) --jw;
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
    int s = seq_id[row];
    return s < 0 ? 0 : (s >= n_seqs ? n_seqs - 1 : s);
  }
  __device__ __forceinline__ int pos_of(int row) const {
    int t = pos[row];
    return t < 0 ? 0 : (t > max_pos ? max_pos : t);
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
  int materialize;       // long rows keep their scores in ws_scores
  float* ws_scores;      // [R][ws_ld]
  int64_t ws_ld;
  uint32_t* cnt_a;       // [R]
  uint32_t* cnt_b;       // [R]
  uint32_t* flags;       // [R]
  uint32_t* tau;         // [R]
  uint32_t* chunk_cnt;   // [R][w_max]
  uint32_t* tops;        // [R][kUnionCap]
  uint2* slots;          // [R][kSlotCap]
};

void run_pool(const PoolArgs& a, int dtype, int di, int n_seqs, hipStream_t st);
void run_scores(const IdxArgs& a, int dtype, int di, int n_rows, int max_n, float* scores,
                int64_t ld, hipStream_t st);
void run_topk(const TopkArgs& t, int dtype, int di, int rows, hipStream_t st);

}  // namespace qsa
