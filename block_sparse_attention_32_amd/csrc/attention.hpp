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
int attn_tile_tokens(int dtype, int hq, int hkv, int d);
void run_attention(const AttnArgs& a, int dtype, int d, bool dense, int n_rows, hipStream_t st);

}  // namespace qsa

namespace qsa {

// MFMA path (bfloat16, head_dim 64 or 128, up to 16 query heads per KV
// head, 1, 2 or 4 KV heads): tile geometry.
constexpr int kMfmaTileTok = 16;    // tokens per wave tile
constexpr int kMfmaTileEnt = 4;     // token-list entries (blocks) per tile
constexpr int kMfmaSplitEnt = 16;   // entries per split and KV head (split-K decode)
constexpr int kMfmaEntChunk = 512;  // entries staged in LDS per pass

bool attn_mfma_supported(int dtype, int hq, int hkv, int d);
void run_attention_mfma(const AttnArgs& a, int d, bool dense, int n_rows, hipStream_t st);

// Dense causal flash attention for many rows (dense_prefill.hip): bfloat16,
// head_dim 64 or 128, Hq/Hkv dividing 16.
bool dense_flash_supported(int dtype, int hq, int hkv, int d);
void run_dense_flash(const AttnArgs& a, int d, int n_rows, hipStream_t st);

}  // namespace qsa
