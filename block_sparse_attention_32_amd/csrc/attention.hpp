// Argument block and host entry points of the attention kernels.
#pragma once

#include "common.hpp"

namespace qsa {

constexpr int kAttnThreads = 256;
constexpr int kMaxOutPerThread = 16;   // n_q_heads * head_dim <= 4096
constexpr int kAttnLds = 64 * 1024;    // dynamic LDS budget of the generic kernel

struct AttnArgs {
  PageMap pm;
  const void* k;
  const void* v;
  int hkv, hq;
  const void* q;          // [T][hq][D]
  void* out;              // [T][hq][D]
  const int32_t* seq_id;
  const int32_t* pos;
  int n_seqs;             // seq_id is clamped to [0, n_seqs)
  int max_pos;            // pos is clamped to [0, max_pos]
  const int32_t* sel;     // [T][top_k] (sparse)
  const int32_t* n_sel;   // [T]
  int top_k;
  float scale;
  int n_splits;           // workgroups per row
  int eps;                // token-list entries (blocks) per split
  int tile_tokens;        // tokens staged per tile (multiple of 4)
  float* part_acc;        // [T][n_splits][hq][D]
  float* part_ml;         // [T][n_splits][hq][2]
  uint32_t* cnt;          // [T]
  int64_t n_slots;        // token rows of the K and V arrays (pages x page size)
  const int32_t* sel_of;  // [T] or null: row i reuses the selection of row sel_of[i]
  int n_rows;             // T
};

// A row reusing another row's selection attends at most this many whole
// blocks between that row's own block and its own (QSA_MAX_SHARED_LAG
// tokens: as many blocks at block size 1).
constexpr int kMaxBridge = QSA_MAX_SHARED_LAG;

// The block list of one row: n_list selected entries, then n_bridge whole
// blocks b_sel .. b_own - 1, then the own block (the last entry).  Selected
// ids outside [0, b_sel) are skipped.
struct RowList {
  int b_own, b_sel, n_list, n_bridge, e_own;
  bool own_sel;  // the row's own selection (not another row's)
  const int32_t* sel;
  // n_sel_row: n_sel[row] (the caller reads it beside the row's other
  // values, so that the reads overlap)
  __device__ __forceinline__ RowList(const AttnArgs& a, int row, int t, bool dense,
                                     int n_sel_row) {
    const int bs = a.pm.blk_shift;
    b_own = t >> bs;
    int rs = row;
    b_sel = b_own;
    n_list = dense ? b_own : clamp_flag(n_sel_row, 0, a.top_k, QSA_DEBUG_BAD_SEL);
    if (!dense && a.sel_of != nullptr) {
      rs = clamp_flag(a.sel_of[row], 0, a.n_rows - 1, QSA_DEBUG_BAD_SEL);
      const int ts = min(max(a.pos[rs], 0), a.max_pos);
      b_sel = max(min(ts >> bs, b_own), b_own - (((QSA_MAX_SHARED_LAG - 1) >> bs) + 1));
      if (rs != row) n_list = clamp_flag(a.n_sel[rs], 0, a.top_k, QSA_DEBUG_BAD_SEL);
    }
    own_sel = rs == row;
    n_bridge = b_own - b_sel;
    e_own = n_list + n_bridge;
    sel = dense ? nullptr : a.sel + (int64_t)rs * a.top_k;
  }
  // block of entry e (< e_own) and whether it is attended
  __device__ __forceinline__ int block(int e, bool dense, bool& ok) const {
    if (e >= n_list) {
      ok = true;
      return b_sel + (e - n_list);
    }
    const int b = dense ? e : sel[e];
    ok = b >= 0 && b < b_sel;
    if (!ok && own_sel) debug_flag(QSA_DEBUG_BAD_SEL);
    return b;
  }
};

// LDS layout of the generic kernel (byte offsets, each 16-byte aligned).
struct AttnLayout {
  size_t q, s, m, l, c, trow, k, v, total;
};
__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ inline AttnLayout attn_layout(int esz, int hq, int hkv, int d, int tt) {
  AttnLayout L;
  size_t o = 0;
  L.q = o; o = align16(o + (size_t)hq * d * 4);
  L.s = o; o = align16(o + (size_t)hq * tt * 4);
  L.m = o; o = align16(o + (size_t)hq * 4);
  L.l = o; o = align16(o + (size_t)hq * 4);
  L.c = o; o = align16(o + (size_t)hq * 4);
  L.trow = o; o = align16(o + (size_t)tt * 8);
  L.k = o; o = align16(o + (size_t)tt * hkv * d * esz);
  L.v = o; o = align16(o + (size_t)tt * hkv * d * esz);
  L.total = o;
  return L;
}
int attn_tile_tokens(int dtype, int hq, int hkv, int d, int block);
void run_attention(const AttnArgs& a, int dtype, int d, bool dense, int n_rows, hipStream_t st);

}  // namespace qsa

namespace qsa {

// MFMA path (bfloat16, head_dim 64 or 128, up to 16 query heads per KV
// head, 1, 2 or 4 KV heads): tile geometry.
constexpr int kMfmaTileTok = 16;    // tokens per wave tile
constexpr int kMfmaSplitEnt = 16;   // 4-token units per split and KV head (split-K decode)
constexpr int kMfmaListTok = 2048;  // list tokens staged in LDS per pass
// Many-row attention in pairs of rows: each row's list (selection and own
// block) holds at most kPairHalf entries, their union at most kPairCap.
constexpr int kPairHalf = 544;
constexpr int kPairCap = 2 * kPairHalf;

bool attn_mfma_supported(int dtype, int hq, int hkv, int d);
void run_attention_mfma(const AttnArgs& a, int d, bool dense, int n_rows, hipStream_t st);

// Dense causal flash attention for many rows (dense_prefill.hip): bfloat16,
// head_dim 64 or 128, Hq/Hkv dividing 16.
bool dense_flash_supported(int dtype, int hq, int hkv, int d);
void run_dense_flash(const AttnArgs& a, int d, int n_rows, hipStream_t st);

}  // namespace qsa
