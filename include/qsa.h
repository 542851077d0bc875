/*
 * qsa.h -- C ABI of libqsa, the MI355X (gfx950) hot path of Qwen Sparse
 * Attention (QSA).
 *
 * What the calls compute (sources are the web pages describing the method):
 *
 *   - keieiax.jp glossary "Qwen Sparse Attention", section
 *     4トークンずつまとめて、必要な場所を探す: the context is compressed into
 *     4-token micro-blocks; a lightweight learned indexer estimates the
 *     importance of each block; at most 512 blocks (2,048 tokens) are
 *     selected per query.
 *   - blog.cecily.jp/6295 (digest of llama.cpp PR #30965), paragraph on
 *     Raschka's explanation: the indexer averages the keys of each block and
 *     scores it, and blocks are taken best first; paragraph on the trade-offs:
 *     whole blocks are read, and the budget is 2,048 tokens plus the current
 *     fractional block.
 *   - ai-manual.ru, "Экономия VRAM в llama.cpp: что даёт QSA-выбор без
 *     kq_mask", section "QSA-выбор и kq_mask": the selection is consumed
 *     without materialising a [queries x keys] mask.
 *   - ai-manual.ru, "llama.cpp получил разреженный Flash Attention для Qwen4
 *     на CUDA", section "Разреженный Flash Attention и обычный": attention is
 *     computed tile by tile without writing intermediates to global memory,
 *     and the sparse variant drops token pairs.
 *   - keieiax.jp glossary, section 長文AIのコストと応答時間にどう影響する？: the
 *     reference point is dense grouped-query attention (GQA); the dense calls
 *     below provide it on the same cache.
 *   - blog.cecily.jp/6295, paragraph on Raschka's explanation: DeepSeek
 *     Sparse Attention selects single tokens where QSA selects 4-token
 *     blocks; paragraph on the trade-offs: the block index is the coarser
 *     one.  The block size B is therefore a cache parameter: B = 4 is QSA,
 *     B = 1 the token-granular selection (with the same 2,048-token budget,
 *     top_k = 2048 / B), and 2, 8, 16 lie around them.
 *
 * The indexer score is not printed on the pages; this library fixes it as
 *     s[b] = sum_h w[h] * max(0, q_idx[h] . kbar[b])
 * with one indexer key head (dimension Di) shared by all indexer query heads.
 *
 * Conventions shared by every call:
 *   - Ownership: every pointer inside the structs and every array argument
 *     is DEVICE memory owned by the caller, unless marked "host".  The
 *     library never allocates or frees memory and keeps no pointer after a
 *     call returns.
 *   - Execution: every call only enqueues kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream) and returns; it
 *     never synchronises and never copies device data to the host.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; on failure nothing is written and a negative qsa_status is
 *     returned.  QSA_ERR_HIP reports a failed launch (hipGetLastError).
 *     Device-side data (page ids, positions, seq_len, sel) must be in range;
 *     out-of-range device data is undefined behaviour.
 *   - Positions: query row i belongs to sequence seq_id[i] and sits at
 *     absolute position pos[i] (0-based); its own K/V/indexer key is already
 *     in the cache, and it may see tokens 0..pos[i] only.  With B tokens per
 *     block (qsa_cache.block_size) its own block is b_own = pos[i] / B;
 *     blocks 0..b_own-1 are its candidates; the own block's tokens
 *     B*b_own..pos[i] are always attended.
 *   - Workspaces: size them with qsa_workspace_size().  A workspace must be
 *     zero-filled once before its first use; every call leaves its counters
 *     at zero again when its kernels finish, so a workspace can be reused by
 *     later calls on the same stream without clearing.  Calls that share one
 *     workspace must not run concurrently.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_BLOCK 4        /* tokens per micro-block of QSA (block_size 0 means this) */
#define QSA_MAX_BLOCK 16   /* largest supported block_size */
#define QSA_BUDGET_TOKENS 2048 /* the pages' selection budget in tokens */
#define QSA_MAX_TOPK 2048  /* largest supported top_k (the budget at block size 1) */
#define QSA_MAX_BLOCKS (1 << 20) /* candidate blocks per query */
#define QSA_MAX_SHARED_LAG 60    /* qsa_attn_decode_shared: pos[i] - pos[sel_of[i]] */

typedef enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes */
  QSA_ERR_UNSUPPORTED = -2, /* valid, but a shape/dtype the library lacks */
  QSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  QSA_ERR_HIP = -4          /* the HIP runtime reported an error           */
} qsa_status;

typedef enum qsa_dtype { QSA_F32 = 0, QSA_BF16 = 1 } qsa_dtype;

typedef enum qsa_op {
  QSA_OP_TOPK = 0,
  QSA_OP_ATTN_DECODE = 1,
  QSA_OP_ATTN_PREFILL = 2,
  QSA_OP_DENSE_DECODE = 3,
  QSA_OP_DENSE_PREFILL = 4,
  QSA_OP_ATTN_DECODE_SHARED = 5
} qsa_op;

/* Paged cache shared by K, V, the indexer keys and the pooled block keys.
 * Logical token j of sequence s lives in physical page
 * block_table[s * max_pages_per_seq + j / page_size], slot j % page_size. */
typedef struct qsa_cache {
  int32_t dtype;             /* qsa_dtype of k, v, kidx, kbar, q, q_idx, out */
  int32_t page_size;         /* tokens per page: a power of two, >= 4 and >= B */
  int32_t block_size;        /* B, tokens per pooled block: 1, 2, 4, 8 or 16;
                                0 means QSA_BLOCK (4)                        */
  int32_t n_kv_heads;        /* Hkv                                          */
  int32_t head_dim;          /* D: 32, 64 or 128                             */
  int32_t idx_dim;           /* Di: 16, 32, 64 or 128                        */
  int32_t n_seqs;            /* rows of block_table / entries of seq_len     */
  int32_t max_pages_per_seq; /* row stride of block_table                    */
  int32_t max_seq_len;       /* host: upper bound of every seq_len[s]        */
  int64_t n_pages;           /* host: pages in the pool (k, v, kidx, kbar)   */
  const int32_t *block_table;/* [n_seqs][max_pages_per_seq] physical pages   */
  const int32_t *seq_len;    /* [n_seqs] tokens present in the cache         */
  const void *k;             /* [n_pages][page_size][Hkv][D]                 */
  const void *v;             /* [n_pages][page_size][Hkv][D]                 */
  const void *kidx;          /* [n_pages][page_size][Di]   indexer keys      */
  void *kbar;                /* [n_pages][page_size/B][Di] pooled keys       */
} qsa_cache;

/* Query rows of one call. */
typedef struct qsa_queries {
  int32_t n_rows;            /* host: T                                       */
  int32_t max_pos;           /* host: upper bound of every pos[i]             */
  const int32_t *seq_id;     /* [T] sequence of each row                      */
  const int32_t *pos;        /* [T] absolute position of each row             */
} qsa_queries;

/* Step 1 -- pooling (glossary: 4-token micro-blocks; PR #30965 digest:
 * the indexer averages the keys of each block).
 * For every sequence s, for the complete blocks b with
 *   blk_begin[s] <= b < min(seq_len[s] / B, blk_begin[s] + max_new_blocks),
 * writes kbar[b] = ((kidx[Bb] + kidx[Bb+1]) + ... + kidx[Bb+B-1]) / B,
 * summed left to right in float32 and rounded to nearest-even in the cache
 * dtype (for B = 1, the key itself).
 * blk_begin: [n_seqs] device.  max_new_blocks (host) bounds the launch; 0 is
 * a no-op. */
qsa_status qsa_pool_blocks(const qsa_cache *c, const int32_t *blk_begin,
                           int32_t max_new_blocks, void *stream);

/* Step 2 -- indexer scores (glossary: the indexer rates every block).
 * For every row i and candidate block b < pos[i] / B:
 *   scores[i * ld + b] = sum_h w[i*Hi + h] * max(0, q_idx[i][h] . kbar[b])
 * accumulated in float32 (a -0 result is stored as +0).  Columns >= pos[i]/B
 * are not written.  q_idx: [T][Hi][Di] in the cache dtype; w: [T][Hi]
 * float32; 1 <= n_idx_heads <= 8; ld >= max_pos / B (host). */
qsa_status qsa_index_scores(const qsa_cache *c, const qsa_queries *qm,
                            const void *q_idx, const float *w,
                            int32_t n_idx_heads, float *scores, int64_t ld,
                            void *stream);

/* Step 3 -- top-k block selection (glossary: at most 512 blocks per query,
 * best first).  For every row i with n = pos[i] / B candidates:
 *   n_sel[i] = min(top_k, n);
 *   sel[i * top_k + j], j < n_sel[i]: the ids of the n_sel[i] highest scores,
 *       ties broken toward the lower block id, written in ascending order;
 *   sel[i * top_k + j], j >= n_sel[i]: -1.
 * Score source: if scores != NULL they are read from scores[i * ld + b]
 * (as written by qsa_index_scores); if scores == NULL (fused mode) they are
 * computed from q_idx, w and kbar as in qsa_index_scores, and q_idx, w,
 * n_idx_heads must be given.  1 <= top_k <= QSA_MAX_TOPK (the pages'
 * budget is 2048 / B).  Selections of more than 512 blocks of rows with
 * fewer than about 64 K candidates take an exact but slower path.
 * ws: workspace of qsa_workspace_size(QSA_OP_TOPK, ...) bytes, zero-filled
 * before the first call; every call leaves it ready for the next call of
 * the same shape.  Fused calls of 64 rows or more on bfloat16 keys of
 * Di 64 or 128 run the matrix-core indexer, whose data lies over the
 * chunked path's counters; such a call zeroes those counters for its own
 * row count and length, so a workspace that then serves a chunked call of
 * other shapes must be zero-filled again first. */
qsa_status qsa_topk_blocks(const qsa_cache *c, const qsa_queries *qm,
                           const float *scores, int64_t ld,
                           const void *q_idx, const float *w,
                           int32_t n_idx_heads, int32_t top_k, int32_t *sel,
                           int32_t *n_sel, void *ws, size_t ws_bytes,
                           void *stream);

/* Steps 1 and 3 fused for a decode step (glossary: the keys of each block
 * are averaged, then the indexer rates every block): for every row i with
 * pos[i] >= B, block pos[i]/B - 1 of sequence seq_id[i] -- the newest
 * complete block before the query -- is pooled into kbar exactly as
 * qsa_pool_blocks would, then the row's selection is made as by
 * qsa_topk_blocks in fused mode (scores computed from q_idx, w, kbar).
 * Precondition: every other block that a row of the call scores is pooled
 * already; in a decode step the sequence's newest block is the only one
 * pooled here.  Rows of one sequence may pool the same block: they write
 * identical values.  Arguments, layouts, workspace and errors as
 * qsa_topk_blocks with scores == NULL; also QSA_ERR_INVALID_ARG when the
 * cache has no kidx. */
qsa_status qsa_topk_blocks_pool_newest(const qsa_cache *c,
                                       const qsa_queries *qm,
                                       const void *q_idx, const float *w,
                                       int32_t n_idx_heads, int32_t top_k,
                                       int32_t *sel, int32_t *n_sel, void *ws,
                                       size_t ws_bytes, void *stream);

/* Steps 4/5 -- block-sparse attention without a mask (PR #30965 digest:
 * whole selected blocks plus the current fractional block; sparse FA
 * explainer: tiled softmax attention).  For every row i and query head hq
 * (KV head hk = hq / (n_q_heads / Hkv)), over the token set
 *   S_i = {Bb .. Bb+B-1 : b in sel[i][0 .. n_sel[i]-1]} U {B*(pos[i]/B) .. pos[i]}
 *   out[i][hq] = sum_{j in S_i} softmax_j(scale * q[i][hq] . K[j][hk]) V[j][hk]
 * accumulated in float32 and rounded to nearest-even in the cache dtype.
 * q, out: [T][n_q_heads][D] in the cache dtype; sel/n_sel as written by
 * qsa_topk_blocks (row stride top_k).  Ids outside [0, pos[i]/B) among
 * the first n_sel[i] entries are skipped.
 * qsa_attn_decode splits each row's token set across workgroups (for few
 * rows); qsa_attn_prefill gives each row its own workgroup (for many rows).
 * Both compute the same result. */
qsa_status qsa_attn_decode(const qsa_cache *c, const qsa_queries *qm,
                           const void *q, int32_t n_q_heads,
                           const int32_t *sel, const int32_t *n_sel,
                           int32_t top_k, float scale, void *out, void *ws,
                           size_t ws_bytes, void *stream);
qsa_status qsa_attn_prefill(const qsa_cache *c, const qsa_queries *qm,
                            const void *q, int32_t n_q_heads,
                            const int32_t *sel, const int32_t *n_sel,
                            int32_t top_k, float scale, void *out, void *ws,
                            size_t ws_bytes, void *stream);

/* qsa_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation): computes exactly what qsa_attn_decode computes, with
 * the same kernels, using a static scratch array of
 * QSA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  It calls no hipMalloc/hipFree.  Arguments,
 * layouts and errors as qsa_attn_decode, plus QSA_ERR_WORKSPACE when the
 * call's plan needs more than the scratch holds (never for head_dim <= 128
 * and n_q_heads <= 16 on the matrix-core path, whose workgroups are capped
 * at 1,024), QSA_ERR_HIP when the scratch's address cannot be obtained.
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from different threads) race and must be
 * serialised by the caller. */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)
qsa_status qsa_attn_decode_noalloc(const qsa_cache *c, const qsa_queries *qm,
                                   const void *q, int32_t n_q_heads,
                                   const int32_t *sel, const int32_t *n_sel,
                                   int32_t top_k, float scale, void *out,
                                   void *stream);

/* Indexer projections (the input side of the learned indexer the
 * keieiax.jp glossary describes in section 4トークンずつまとめて; the pages
 * print no projection, so these are plain linear maps, no bias).  For every
 * row i (token pos[i] of sequence seq_id[i]) with hidden state x[i]:
 *   q_idx[i][h][d] = bf(sum_c x[i][c] * wq[h*Di + d][c])
 *   kidx_out[token pos[i] of seq_id[i]][d] = bf(sum_c x[i][c] * wk[d][c])
 *   w[i][h] = sum_c x[i][c] * ww[h][c]                       (float32)
 * bf = round to nearest-even bfloat16 of the float32 sum.  x: [T][h_dim];
 * wq: [Hi*Di][h_dim]; wk: [Di][h_dim]; ww: [Hi][h_dim] (each output's
 * weights contiguous); q_idx: [T][Hi][Di]; kidx_out: the paged layout of
 * qsa_cache.kidx (normally that buffer); w: [T][Hi].  bfloat16 caches only;
 * h_dim a positive multiple of 64; 1 <= n_idx_heads <= 8. */
qsa_status qsa_index_project(const qsa_cache *c, const qsa_queries *qm,
                             const void *x, int32_t h_dim, const void *wq,
                             const void *wk, const void *ww,
                             int32_t n_idx_heads, void *q_idx, void *kidx_out,
                             float *w, void *stream);

/* Multi-token decode with one selection reused across draft positions
 * (keieiax.jp glossary, FAQ on whether the selection is shared across
 * layers: multi-token prediction may reuse the top index across its
 * speculative steps).  Row i attends the selection made for row
 * s = sel_of[i] (a row of the same call, same sequence, at position
 * pos[s] <= pos[i] <= pos[s] + QSA_MAX_SHARED_LAG), and everything from the
 * start of that row's own block up to its own position:
 *   S_i = {Bb .. Bb+B-1 : b in sel[s][0 .. n_sel[s]-1], b < pos[s]/B}
 *         U {B*(pos[s]/B) .. pos[i]}
 * sel_of[i] = i gives exactly qsa_attn_decode's result.  sel_of: [T] device
 * int32; rows outside the limits above are clamped to them (their result
 * is unspecified).  sel and n_sel must hold all T rows ([T][top_k] and
 * [T]), also those of rows that reuse another row's selection: every row's
 * own entries are read (and ignored when sel_of[i] != i), so that the reads
 * of a row start together.  ws: qsa_workspace_size(QSA_OP_ATTN_DECODE_SHARED,
 * ...). */
qsa_status qsa_attn_decode_shared(const qsa_cache *c, const qsa_queries *qm,
                                  const void *q, int32_t n_q_heads,
                                  const int32_t *sel, const int32_t *n_sel,
                                  const int32_t *sel_of, int32_t top_k,
                                  float scale, void *out, void *ws,
                                  size_t ws_bytes, void *stream);

/* Comparison baseline (glossary: dense GQA attention kernels): causal
 * attention of every row over all tokens 0..pos[i] of its sequence, same
 * layouts and rounding as the sparse calls. */
qsa_status qsa_dense_attn_decode(const qsa_cache *c, const qsa_queries *qm,
                                 const void *q, int32_t n_q_heads,
                                 float scale, void *out, void *ws,
                                 size_t ws_bytes, void *stream);
qsa_status qsa_dense_attn_prefill(const qsa_cache *c, const qsa_queries *qm,
                                  const void *q, int32_t n_q_heads,
                                  float scale, void *out, void *ws,
                                  size_t ws_bytes, void *stream);

/* Workspace bytes needed by `op` (a qsa_op) for these shapes; host-only,
 * reads only host fields of c and qm.  top_k is ignored by the dense ops,
 * n_q_heads by QSA_OP_TOPK.  Returns 0 for a null argument or unknown op. */
size_t qsa_workspace_size(int32_t op, const qsa_cache *c,
                          const qsa_queries *qm, int32_t n_q_heads,
                          int32_t top_k);

/* Debug builds (libqsa_debug.so, compiled with -DQSA_DEBUG): the kernels
 * check the device data the host cannot -- page ids read from block_table,
 * sequence ids and positions, selection lengths and selected ids -- and
 * replace an out-of-range value with one that keeps every access inside
 * the caller's buffers (page 0; the clamped id or position; the selection
 * entry skipped), recording what they saw in these bits: */
#define QSA_DEBUG_BAD_PAGE 1u /* a block_table entry outside [0, n_pages)         */
#define QSA_DEBUG_BAD_ROW  2u /* seq_id outside [0, n_seqs) or pos outside
                                 [0, max_pos]                                      */
#define QSA_DEBUG_BAD_SEL  4u /* n_sel outside [0, top_k], a row's selected id
                                 outside [0, pos/B), or sel_of outside [0, T)     */
/* qsa_debug_take: waits for the device (hipDeviceSynchronize), ORs the bits
 * recorded since the last call into *flags (host) and clears them.  For
 * debugging only: it synchronises.  The release build (libqsa.so) records
 * nothing: *flags = 0 and QSA_ERR_UNSUPPORTED.  QSA_ERR_INVALID_ARG for a
 * null flags. */
qsa_status qsa_debug_take(uint32_t *flags);

/* Static description of a status code. */
const char *qsa_status_string(qsa_status s);

/* Library version, (major << 16) | minor. */
int32_t qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
