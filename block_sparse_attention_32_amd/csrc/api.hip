// C ABI of libqsa: host-side validation, workspace planning and launches.
// Every call validates its arguments before enqueuing anything and never
// synchronises, allocates or copies device data to the host.
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "attention.hpp"
#include "project.hpp"
#include "index.hpp"

using namespace qsa;

#ifdef QSA_DEBUG
namespace qsa {
// the error-word readers of every translation unit (registered at load)
static std::vector<uint32_t (*)()>& debug_units() {
  static std::vector<uint32_t (*)()> units;
  return units;
}
void debug_register(uint32_t (*take)()) { debug_units().push_back(take); }
}  // namespace qsa
#endif

namespace {

constexpr int kRowBatch = 4096;              // top-k rows per launch pair
constexpr int kTargetSplitWgs = 256;         // decode (generic kernel): workgroups over all rows
constexpr int kMinEntriesPerSplit = 8;
constexpr int64_t kMaxSplitWgs = 1024;       // decode (MFMA kernel): workgroup cap

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// tokens per pooled block (0 stands for QSA's 4)
int cache_block(const qsa_cache* c) { return c->block_size == 0 ? QSA_BLOCK : c->block_size; }

qsa_status check_cache(const qsa_cache* c) {
  if (c == nullptr) return QSA_ERR_INVALID_ARG;
  if (c->dtype != QSA_F32 && c->dtype != QSA_BF16) return QSA_ERR_INVALID_ARG;
  if (!is_pow2(c->page_size) || c->page_size < 4) return QSA_ERR_INVALID_ARG;
  const int blk = cache_block(c);
  if (!is_pow2(blk) || blk > QSA_MAX_BLOCK || blk > c->page_size) return QSA_ERR_INVALID_ARG;
  if (c->n_kv_heads < 1 || c->n_seqs < 1 || c->max_pages_per_seq < 1) return QSA_ERR_INVALID_ARG;
  if (c->max_seq_len < 1 || c->n_pages < 1) return QSA_ERR_INVALID_ARG;
  if ((int64_t)c->max_seq_len > (int64_t)c->max_pages_per_seq * c->page_size)
    return QSA_ERR_INVALID_ARG;
  if (c->block_table == nullptr || c->seq_len == nullptr) return QSA_ERR_INVALID_ARG;
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return QSA_ERR_UNSUPPORTED;
  if ((int64_t)c->n_pages * c->page_size > INT32_MAX) return QSA_ERR_UNSUPPORTED;  // token rows fit int32
  if (c->idx_dim != 16 && c->idx_dim != 32 && c->idx_dim != 64 && c->idx_dim != 128)
    return QSA_ERR_UNSUPPORTED;
  return QSA_OK;
}

qsa_status check_queries(const qsa_cache* c, const qsa_queries* qm) {
  if (qm == nullptr) return QSA_ERR_INVALID_ARG;
  if (qm->n_rows < 0 || qm->max_pos < 0) return QSA_ERR_INVALID_ARG;
  if (qm->n_rows > 0 && (qm->seq_id == nullptr || qm->pos == nullptr)) return QSA_ERR_INVALID_ARG;
  if (qm->max_pos >= c->max_seq_len) return QSA_ERR_INVALID_ARG;
  if (qm->max_pos / cache_block(c) > QSA_MAX_BLOCKS) return QSA_ERR_UNSUPPORTED;
  if (qm->n_rows > 65535) return QSA_ERR_UNSUPPORTED;  // grid y
  return QSA_OK;
}

PageMap page_map(const qsa_cache* c) {
  PageMap pm;
  pm.table = c->block_table;
  pm.max_pages = c->max_pages_per_seq;
  pm.page_shift = log2i(c->page_size);
  pm.blk_shift = log2i(cache_block(c));
  pm.n_pages = c->n_pages;
  return pm;
}

qsa_status launched() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

// ------------------------------------------------------------- top-k plan

struct TopkPlan {
  int rows, w_max, ucap;
  int64_t ws_ld;
  size_t off_ctr, off_tops, off_nxt, off_scores, total;
};

// MFMA prefill indexer plan (fused mode, many rows)
struct PidxPlan {
  int rows, splits;
  size_t off_uni, off_tau, off_tstride, off_rstride, off_surv, off_scnt, off_done, off_fbcnt,
      off_fblist, total;
};

PidxPlan pidx_plan(const qsa_queries* qm) {
  PidxPlan p;
  p.rows = qm->n_rows < kPRowBatch ? qm->n_rows : kPRowBatch;
  if (p.rows < 1) p.rows = 1;
  const int tiles = (p.rows + kPQT - 1) / kPQT;
  // enough workgroups for two per CU (the scoring kernel's 128 VGPRs per
  // lane allow two of its 8-wave workgroups on a CU)
  int sp = (512 + tiles - 1) / tiles;
  p.splits = sp < 1 ? 1 : (sp > kPMaxSplits ? kPMaxSplits : sp);
  size_t o = 0;
  p.off_uni = o;     o = align256(o + (size_t)p.rows * kPUnion * 4);
  p.off_tau = o;     o = align256(o + (size_t)p.rows * 4);
  p.off_tstride = o; o = align256(o + (size_t)(tiles + 1) * 4);
  p.off_rstride = o; o = align256(o + (size_t)p.rows * 4);
  p.off_surv = o;    o = align256(o + (size_t)p.rows * kPSurvCap * 8);
  p.off_scnt = o;    o = align256(o + (size_t)p.rows * p.splits * 4);
  p.off_done = o;    o = align256(o + (size_t)p.rows * 4);
  p.off_fbcnt = o;   o = align256(o + 2 * 4);
  p.off_fblist = o;  o = align256(o + (size_t)p.rows * 4);
  p.total = o;
  return p;
}

TopkPlan topk_plan(const qsa_cache* c, const qsa_queries* qm, int top_k) {
  TopkPlan p;
  const int max_n = qm->max_pos / cache_block(c);
  p.w_max = (max_n + kChunk - 1) / kChunk;
  if (p.w_max < 1) p.w_max = 1;
  p.ucap = union_cap(top_k, p.w_max);
  // rows per launch (fewer for the wider unions)
  const int batch = kRowBatch * kUnionCap / p.ucap;
  p.rows = qm->n_rows < batch ? qm->n_rows : batch;
  if (p.rows < 1) p.rows = 1;
  // rows of at most kDirectCap candidates keep their keys for the exact
  // select; longer rows keep none (a rare rescan recomputes its keys)
  const int64_t full = (int64_t)p.w_max * kChunk;
  p.ws_ld = full < kDirectCap ? full : kDirectCap;
  size_t o = 0;
  p.off_ctr = o;    o = align256(o + (size_t)p.rows * arrive_slots(p.w_max) * kCtrStride * 4);
  p.off_tops = o;   o = align256(o + (size_t)p.rows * p.ucap * 8);
  p.off_nxt = o;    o = align256(o + (size_t)p.rows * p.w_max * kChunkWaves * 4);
  p.off_scores = o; o = align256(o + (size_t)p.rows * p.ws_ld * 4);
  p.total = o;
  return p;
}

// ------------------------------------------------------------- attention plan

struct AttnPlan {
  int splits, eps, tile, mfma;
  size_t off_cnt, off_ml, off_acc, total;
};

AttnPlan attn_plan(int op, const qsa_cache* c, const qsa_queries* qm, int hq, int top_k) {
  AttnPlan p;
  const bool dense = (op == QSA_OP_DENSE_DECODE || op == QSA_OP_DENSE_PREFILL);
  const bool split = (op == QSA_OP_ATTN_DECODE || op == QSA_OP_DENSE_DECODE ||
                     op == QSA_OP_ATTN_DECODE_SHARED);
  // a row reusing another row's selection also attends up to
  // ceil(QSA_MAX_SHARED_LAG / B) whole blocks before its own
  const int blk = cache_block(c);
  const int entries = (dense ? qm->max_pos / blk : top_k) + 1 +
                      (op == QSA_OP_ATTN_DECODE_SHARED ? (QSA_MAX_SHARED_LAG + blk - 1) / blk : 0);
  p.mfma = attn_mfma_supported(c->dtype, hq, c->n_kv_heads, c->head_dim) ? 1 : 0;
  p.tile = p.mfma ? kMfmaTileTok
                  : attn_tile_tokens(c->dtype, hq, c->n_kv_heads, c->head_dim, blk);
  const int rows = qm->n_rows > 0 ? qm->n_rows : 1;
  if (split && p.mfma) {
    // Planned in 4-token units (one QSA block), then converted to entries.
    // Split workgroups have 8 waves, wph of them per KV head, and each
    // wave gets two 16-token tiles (kMfmaSplitEnt = 16 units per wave
    // pair); grow the split when rows x splits would exceed kMaxSplitWgs
    const int units = (int)(((int64_t)entries * blk + 3) / 4);
    const int wph = 8 / c->n_kv_heads;
    int eps = kMfmaSplitEnt * wph / 2;
    // a row's last split merges up to 16 partials in one round trip: when a
    // few more units per split (at most a quarter) bring the count to 16,
    // take them
    const int e16 = ((units + 15) / 16 + 3) / 4 * 4;
    if ((units + eps - 1) / eps > 16 && e16 * 4 <= eps * 5) eps = e16;
    while ((int64_t)rows * ((units + eps - 1) / eps) > kMaxSplitWgs) eps *= 2;
    p.eps = eps * 4 / blk > 0 ? eps * 4 / blk : 1;
    p.splits = (entries + p.eps - 1) / p.eps;
  } else if (split) {
    int s = (kTargetSplitWgs + rows - 1) / rows;
    int s_max = (entries + kMinEntriesPerSplit - 1) / kMinEntriesPerSplit;
    if (s > s_max) s = s_max;
    if (s < 1) s = 1;
    p.eps = (entries + s - 1) / s;
    p.splits = (entries + p.eps - 1) / p.eps;
  } else {
    p.splits = 1;
    p.eps = entries;
  }
  size_t o = 0;
  p.off_cnt = o;
  p.off_ml = p.off_acc = 0;
  if (p.splits > 1) {
    o = align256(o + (size_t)rows * 4);
    p.off_ml = o;  o = align256(o + (size_t)rows * p.splits * hq * 2 * 4);
    p.off_acc = o; o = align256(o + (size_t)rows * p.splits * hq * c->head_dim * 4);
  }
  p.total = o;
  return p;
}

// ------------------------------------------------------------- static scratch

// The workspace of qsa_attn_decode_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: each device's address is looked up once,
// with that device current, and kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* scratch_addr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];
std::once_flag scratch_once[kMaxDevices];

// the current device's copy of `scratch`
qsa_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QSA_ERR_UNSUPPORTED;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_addr[dev] = p;
  });
  if (scratch_err[dev] != hipSuccess || scratch_addr[dev] == nullptr) return QSA_ERR_HIP;
  *out = scratch_addr[dev];
  return QSA_OK;
}

// zeroes n 32-bit words (a kernel, not a memset, so that graph capture
// records a kernel node)
__global__ void __launch_bounds__(256) clear_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

qsa_status attention_common(int op, const qsa_cache* c, const qsa_queries* qm, const void* q,
                            int32_t hq, const int32_t* sel, const int32_t* n_sel,
                            int32_t top_k, float scale, void* out, void* ws, size_t ws_bytes,
                            void* stream, const int32_t* sel_of = nullptr,
                            bool use_scratch = false) {
  qsa_status st = check_cache(c);
  if (st != QSA_OK) return st;
  if ((st = check_queries(c, qm)) != QSA_OK) return st;
  const bool dense = (op == QSA_OP_DENSE_DECODE || op == QSA_OP_DENSE_PREFILL);
  if (hq < 1 || hq % c->n_kv_heads != 0) return QSA_ERR_INVALID_ARG;
  if (hq * c->head_dim > kMaxOutPerThread * kAttnThreads) return QSA_ERR_UNSUPPORTED;
  if (!dense && (top_k < 1 || top_k > QSA_MAX_TOPK)) return QSA_ERR_INVALID_ARG;
  if (!dense && (sel == nullptr || n_sel == nullptr)) return QSA_ERR_INVALID_ARG;
  if (op == QSA_OP_ATTN_DECODE_SHARED && sel_of == nullptr) return QSA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || scale != scale) return QSA_ERR_INVALID_ARG;
  if (qm->n_rows > 0 && (q == nullptr || out == nullptr)) return QSA_ERR_INVALID_ARG;
  if (c->k == nullptr || c->v == nullptr) return QSA_ERR_INVALID_ARG;
  const AttnPlan p = attn_plan(op, c, qm, hq, top_k);
  if (p.tile < 4) return QSA_ERR_UNSUPPORTED;
  if (use_scratch) {
    // the static scratch replaces the caller's workspace
    if (p.total > QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_WORKSPACE;
    if (qm->n_rows == 0) return QSA_OK;
    if ((st = scratch_for_current_device(&ws)) != QSA_OK) return st;
    ws_bytes = QSA_NOALLOC_SCRATCH_BYTES;
    if (p.splits > 1) {
      // the arrival counters start at zero (the array keeps the last
      // call's contents)
      hipLaunchKernelGGL(clear_words, dim3((unsigned)((qm->n_rows + 255) / 256)), dim3(256), 0,
                         as_stream(stream),
                         reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + p.off_cnt),
                         qm->n_rows);
      if ((st = launched()) != QSA_OK) return st;
    }
  }
  if (p.total > 0 && (ws == nullptr || ws_bytes < p.total)) return QSA_ERR_WORKSPACE;
  if (qm->n_rows == 0) return QSA_OK;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.pm = page_map(c);
  a.k = c->k;
  a.v = c->v;
  a.n_slots = (int64_t)c->n_pages * c->page_size;
  a.hkv = c->n_kv_heads;
  a.hq = hq;
  a.q = q;
  a.out = out;
  a.seq_id = qm->seq_id;
  a.pos = qm->pos;
  a.n_seqs = c->n_seqs;
  a.max_pos = qm->max_pos;
  a.sel = sel;
  a.n_sel = n_sel;
  a.sel_of = sel_of;
  a.n_rows = qm->n_rows;
  a.top_k = top_k;
  a.scale = scale;
  a.n_splits = p.splits;
  a.eps = p.eps;
  a.tile_tokens = p.tile;
  if (p.splits > 1) {
    char* base = static_cast<char*>(ws);
    a.cnt = reinterpret_cast<uint32_t*>(base + p.off_cnt);
    a.part_ml = reinterpret_cast<float*>(base + p.off_ml);
    a.part_acc = reinterpret_cast<float*>(base + p.off_acc);
  }
  if (op == QSA_OP_DENSE_PREFILL &&
      dense_flash_supported(c->dtype, hq, c->n_kv_heads, c->head_dim))
    run_dense_flash(a, c->head_dim, qm->n_rows, as_stream(stream));
  else if (p.mfma)
    run_attention_mfma(a, c->head_dim, dense, qm->n_rows, as_stream(stream));
  else
    run_attention(a, c->dtype, c->head_dim, dense, qm->n_rows, as_stream(stream));
  return launched();
}

}  // namespace

extern "C" {

qsa_status qsa_pool_blocks(const qsa_cache* c, const int32_t* blk_begin, int32_t max_new_blocks,
                           void* stream) {
  qsa_status st = check_cache(c);
  if (st != QSA_OK) return st;
  if (max_new_blocks < 0) return QSA_ERR_INVALID_ARG;
  if (max_new_blocks == 0) return QSA_OK;
  if (blk_begin == nullptr || c->kidx == nullptr || c->kbar == nullptr) return QSA_ERR_INVALID_ARG;
  if (c->n_seqs > 65535) return QSA_ERR_UNSUPPORTED;
  PoolArgs a;
  a.pm = page_map(c);
  a.kidx = c->kidx;
  a.kbar = c->kbar;
  a.seq_len = c->seq_len;
  a.blk_begin = blk_begin;
  a.max_new = max_new_blocks;
  a.max_seq_len = c->max_seq_len;
  run_pool(a, c->dtype, c->idx_dim, c->n_seqs, as_stream(stream));
  return launched();
}

qsa_status qsa_index_scores(const qsa_cache* c, const qsa_queries* qm, const void* q_idx,
                            const float* w, int32_t n_idx_heads, float* scores, int64_t ld,
                            void* stream) {
  qsa_status st = check_cache(c);
  if (st != QSA_OK) return st;
  if ((st = check_queries(c, qm)) != QSA_OK) return st;
  if (n_idx_heads < 1 || n_idx_heads > kMaxIdxHeads) return QSA_ERR_INVALID_ARG;
  const int max_n = qm->max_pos / cache_block(c);
  if (ld < (int64_t)max_n) return QSA_ERR_INVALID_ARG;
  if (qm->n_rows == 0 || max_n == 0) return QSA_OK;
  if (q_idx == nullptr || w == nullptr || scores == nullptr || c->kbar == nullptr)
    return QSA_ERR_INVALID_ARG;
  IdxArgs a;
  a.pm = page_map(c);
  a.kbar = c->kbar;
  a.q_idx = q_idx;
  a.w = w;
  a.hi = n_idx_heads;
  a.seq_id = qm->seq_id;
  a.pos = qm->pos;
  a.n_seqs = c->n_seqs;
  a.max_pos = qm->max_pos;
  run_scores(a, c->dtype, c->idx_dim, qm->n_rows, max_n, scores, ld, as_stream(stream));
  return launched();
}

// qsa_topk_blocks, and with pool_newest its variant that first pools each
// row's newest complete block (fused scoring only)
static qsa_status topk_common(const qsa_cache* c, const qsa_queries* qm, const float* scores,
                              int64_t ld, const void* q_idx, const float* w,
                              int32_t n_idx_heads, int32_t top_k, int32_t* sel,
                              int32_t* n_sel, void* ws, size_t ws_bytes, void* stream,
                              bool pool_newest) {
  qsa_status st = check_cache(c);
  if (st != QSA_OK) return st;
  if ((st = check_queries(c, qm)) != QSA_OK) return st;
  if (top_k < 1 || top_k > QSA_MAX_TOPK) return QSA_ERR_INVALID_ARG;
  if (pool_newest && (scores != nullptr || c->kidx == nullptr)) return QSA_ERR_INVALID_ARG;
  const int max_n = qm->max_pos / cache_block(c);
  if (scores != nullptr) {
    if (ld < (int64_t)max_n) return QSA_ERR_INVALID_ARG;
  } else {
    if (q_idx == nullptr || w == nullptr || c->kbar == nullptr) return QSA_ERR_INVALID_ARG;
    if (n_idx_heads < 1 || n_idx_heads > kMaxIdxHeads) return QSA_ERR_INVALID_ARG;
  }
  if (qm->n_rows > 0 && (sel == nullptr || n_sel == nullptr)) return QSA_ERR_INVALID_ARG;
  const TopkPlan p = topk_plan(c, qm, top_k);
  const PidxPlan pp = pidx_plan(qm);
  const bool mfma = scores == nullptr && qm->n_rows >= kPMinRows &&
                    pidx_supported(c->dtype, c->idx_dim, n_idx_heads);
  // the documented size (qsa_workspace_size) covers both paths; anything
  // smaller is rejected whichever path the call takes
  const size_t need = p.total > pp.total ? p.total : pp.total;
  if (ws == nullptr || ws_bytes < need) return QSA_ERR_WORKSPACE;
  if (qm->n_rows == 0) return QSA_OK;
  char* base = static_cast<char*>(ws);
  if (mfma) {
    PIdxArgs a;
    memset(&a, 0, sizeof(a));
    a.idx.pm = page_map(c);
    a.idx.kbar = c->kbar;
    a.idx.q_idx = q_idx;
    a.idx.w = w;
    a.idx.hi = n_idx_heads;
    a.idx.seq_id = qm->seq_id;
    a.idx.pos = qm->pos;
    a.idx.n_seqs = c->n_seqs;
    a.idx.max_pos = qm->max_pos;
    a.top_k = top_k;
    a.splits = pp.splits;
    a.uni = reinterpret_cast<uint32_t*>(base + pp.off_uni);
    a.tau = reinterpret_cast<uint32_t*>(base + pp.off_tau);
    a.tile_stride = reinterpret_cast<int32_t*>(base + pp.off_tstride);
    a.row_stride = reinterpret_cast<int32_t*>(base + pp.off_rstride);
    a.surv = reinterpret_cast<uint64_t*>(base + pp.off_surv);
    a.surv_cnt = reinterpret_cast<uint32_t*>(base + pp.off_scnt);
    a.done = reinterpret_cast<uint32_t*>(base + pp.off_done);
    a.fb_cnt = reinterpret_cast<uint32_t*>(base + pp.off_fbcnt);
    a.fb_list = reinterpret_cast<int32_t*>(base + pp.off_fblist);
    a.sel = sel;
    a.n_sel = n_sel;
    if (pool_newest) {
      run_pool_rows(a.idx, c->kidx, c->dtype, c->idx_dim, qm->n_rows, as_stream(stream));
      if ((st = launched()) != QSA_OK) return st;
    }
    for (int r0 = 0; r0 < qm->n_rows; r0 += pp.rows) {
      a.row0 = r0;
      a.rows = (qm->n_rows - r0) < pp.rows ? (qm->n_rows - r0) : pp.rows;
      a.idx.seq_id = qm->seq_id;
      run_pidx(a, c->idx_dim, as_stream(stream));
      if ((st = launched()) != QSA_OK) return st;
    }
    // the chunked top-k's arrival counters (the first p.off_tops bytes of
    // its layout) lie under the indexer's data: zero them, so that a later
    // call of the same shape on the chunked path finds them at zero
    const int words = (int)(p.off_tops / 4);
    hipLaunchKernelGGL(clear_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                       as_stream(stream), reinterpret_cast<uint32_t*>(base), words);
    return launched();
  }
  TopkArgs t;
  memset(&t, 0, sizeof(t));
  t.idx.pm = page_map(c);
  t.idx.kbar = c->kbar;
  t.idx.q_idx = q_idx;
  t.idx.w = w;
  t.idx.hi = n_idx_heads;
  t.idx.seq_id = qm->seq_id;
  t.idx.pos = qm->pos;
  t.idx.n_seqs = c->n_seqs;
  t.idx.max_pos = qm->max_pos;
  t.scores = scores;
  t.ld = ld;
  t.top_k = top_k;
  t.sel = sel;
  t.n_sel = n_sel;
  t.w_max = p.w_max;
  t.ws_scores = reinterpret_cast<float*>(base + p.off_scores);
  t.ws_ld = p.ws_ld;
  t.cnt = reinterpret_cast<uint32_t*>(base + p.off_ctr);
  t.ctr_slots = arrive_slots(p.w_max);
  t.tops = reinterpret_cast<uint64_t*>(base + p.off_tops);
  t.nxt = reinterpret_cast<uint32_t*>(base + p.off_nxt);
  t.ucap = p.ucap;
  t.pool_kidx = pool_newest ? c->kidx : nullptr;
  for (int r0 = 0; r0 < qm->n_rows; r0 += p.rows) {
    const int rows = (qm->n_rows - r0) < p.rows ? (qm->n_rows - r0) : p.rows;
    t.row0 = r0;
    run_topk(t, c->dtype, c->idx_dim, rows, as_stream(stream));
    if ((st = launched()) != QSA_OK) return st;
  }
  return QSA_OK;
}

qsa_status qsa_topk_blocks(const qsa_cache* c, const qsa_queries* qm, const float* scores,
                           int64_t ld, const void* q_idx, const float* w, int32_t n_idx_heads,
                           int32_t top_k, int32_t* sel, int32_t* n_sel, void* ws,
                           size_t ws_bytes, void* stream) {
  return topk_common(c, qm, scores, ld, q_idx, w, n_idx_heads, top_k, sel, n_sel, ws, ws_bytes,
                     stream, false);
}

qsa_status qsa_topk_blocks_pool_newest(const qsa_cache* c, const qsa_queries* qm,
                                       const void* q_idx, const float* w, int32_t n_idx_heads,
                                       int32_t top_k, int32_t* sel, int32_t* n_sel, void* ws,
                                       size_t ws_bytes, void* stream) {
  return topk_common(c, qm, nullptr, 0, q_idx, w, n_idx_heads, top_k, sel, n_sel, ws, ws_bytes,
                     stream, true);
}

qsa_status qsa_attn_decode(const qsa_cache* c, const qsa_queries* qm, const void* q,
                           int32_t n_q_heads, const int32_t* sel, const int32_t* n_sel,
                           int32_t top_k, float scale, void* out, void* ws, size_t ws_bytes,
                           void* stream) {
  return attention_common(QSA_OP_ATTN_DECODE, c, qm, q, n_q_heads, sel, n_sel, top_k, scale,
                          out, ws, ws_bytes, stream);
}

qsa_status qsa_attn_decode_noalloc(const qsa_cache* c, const qsa_queries* qm, const void* q,
                                   int32_t n_q_heads, const int32_t* sel, const int32_t* n_sel,
                                   int32_t top_k, float scale, void* out, void* stream) {
  return attention_common(QSA_OP_ATTN_DECODE, c, qm, q, n_q_heads, sel, n_sel, top_k, scale,
                          out, nullptr, 0, stream, nullptr, true);
}

qsa_status qsa_index_project(const qsa_cache* c, const qsa_queries* qm, const void* x,
                             int32_t h_dim, const void* wq, const void* wk, const void* ww,
                             int32_t n_idx_heads, void* q_idx, void* kidx_out, float* w,
                             void* stream) {
  qsa_status st = check_cache(c);
  if (st != QSA_OK) return st;
  if ((st = check_queries(c, qm)) != QSA_OK) return st;
  if (c->dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
  if (n_idx_heads < 1 || n_idx_heads > kMaxIdxHeads) return QSA_ERR_INVALID_ARG;
  if (h_dim < 1 || h_dim % kProjKStep != 0) return QSA_ERR_INVALID_ARG;
  if (qm->n_rows == 0) return QSA_OK;
  if (x == nullptr || wq == nullptr || wk == nullptr || ww == nullptr || q_idx == nullptr ||
      kidx_out == nullptr || w == nullptr)
    return QSA_ERR_INVALID_ARG;
  ProjArgs a;
  a.pm = page_map(c);
  a.x = static_cast<const bf16_t*>(x);
  a.wq = static_cast<const bf16_t*>(wq);
  a.wk = static_cast<const bf16_t*>(wk);
  a.ww = static_cast<const bf16_t*>(ww);
  a.h = h_dim;
  a.nq = n_idx_heads * c->idx_dim;
  a.nk = c->idx_dim;
  a.n = a.nq + a.nk + n_idx_heads;
  a.rows = qm->n_rows;
  a.seq_id = qm->seq_id;
  a.pos = qm->pos;
  a.n_seqs = c->n_seqs;
  a.max_pos = qm->max_pos;
  a.q_idx = static_cast<bf16_t*>(q_idx);
  a.kidx = static_cast<bf16_t*>(kidx_out);
  a.w = w;
  run_project(a, as_stream(stream));
  return launched();
}

qsa_status qsa_attn_decode_shared(const qsa_cache* c, const qsa_queries* qm, const void* q,
                                  int32_t n_q_heads, const int32_t* sel, const int32_t* n_sel,
                                  const int32_t* sel_of, int32_t top_k, float scale, void* out,
                                  void* ws, size_t ws_bytes, void* stream) {
  return attention_common(QSA_OP_ATTN_DECODE_SHARED, c, qm, q, n_q_heads, sel, n_sel, top_k,
                          scale, out, ws, ws_bytes, stream, sel_of);
}

qsa_status qsa_attn_prefill(const qsa_cache* c, const qsa_queries* qm, const void* q,
                            int32_t n_q_heads, const int32_t* sel, const int32_t* n_sel,
                            int32_t top_k, float scale, void* out, void* ws, size_t ws_bytes,
                            void* stream) {
  return attention_common(QSA_OP_ATTN_PREFILL, c, qm, q, n_q_heads, sel, n_sel, top_k, scale,
                          out, ws, ws_bytes, stream);
}

qsa_status qsa_dense_attn_decode(const qsa_cache* c, const qsa_queries* qm, const void* q,
                                 int32_t n_q_heads, float scale, void* out, void* ws,
                                 size_t ws_bytes, void* stream) {
  return attention_common(QSA_OP_DENSE_DECODE, c, qm, q, n_q_heads, nullptr, nullptr, 0, scale,
                          out, ws, ws_bytes, stream);
}

qsa_status qsa_dense_attn_prefill(const qsa_cache* c, const qsa_queries* qm, const void* q,
                                  int32_t n_q_heads, float scale, void* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  return attention_common(QSA_OP_DENSE_PREFILL, c, qm, q, n_q_heads, nullptr, nullptr, 0, scale,
                          out, ws, ws_bytes, stream);
}

size_t qsa_workspace_size(int32_t op, const qsa_cache* c, const qsa_queries* qm,
                          int32_t n_q_heads, int32_t top_k) {
  if (c == nullptr || qm == nullptr) return 0;
  if (check_cache(c) != QSA_OK || check_queries(c, qm) != QSA_OK) return 0;
  switch (op) {
    case QSA_OP_TOPK: {
      const size_t a = topk_plan(c, qm, top_k).total, b = pidx_plan(qm).total;
      return a > b ? a : b;
    }
    case QSA_OP_ATTN_DECODE:
    case QSA_OP_ATTN_DECODE_SHARED:
    case QSA_OP_ATTN_PREFILL:
    case QSA_OP_DENSE_DECODE:
    case QSA_OP_DENSE_PREFILL:
      if (n_q_heads < 1) return 0;
      return attn_plan(op, c, qm, n_q_heads, top_k < 1 ? 1 : top_k).total;
    default:
      return 0;
  }
}

const char* qsa_status_string(qsa_status s) {
  switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case QSA_ERR_WORKSPACE: return "workspace missing or too small";
    case QSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t qsa_version(void) { return (0 << 16) | 2; }

qsa_status qsa_debug_take(uint32_t* flags) {
  if (flags == nullptr) return QSA_ERR_INVALID_ARG;
  *flags = 0u;
#ifdef QSA_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return QSA_ERR_HIP;
  for (auto take : debug_units()) *flags |= take();
  return QSA_OK;
#else
  return QSA_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
