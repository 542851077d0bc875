// Indexer side of the QSA hot path on gfx950: block pooling and block
// scores (this file); the exact per-query top-k block selection of few rows
// is in topk.hpp, of many rows in index_mfma.hip.
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

#include "index_device.hpp"

namespace qsa {

// the top-k launches, one translation unit per (element type, Di)
template <typename T, int DI>
void launch_topk_typed(const TopkArgs& t, int rows, hipStream_t st);

// ================================================================ pooling

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
    launch_topk_typed<decltype(tag), decltype(dic)::value>(t, rows, st);
  });
}

}  // namespace qsa

