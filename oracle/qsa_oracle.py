"""Plain CPU oracle for Qwen Sparse Attention (QSA) selection and attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The GPU library never
calls it, links it or falls back to it, and it shares no code with the GPU
library: it is numpy in float64, written step by step from the method's
description so that it can be checked by eye.

Sources (the web pages this method is described on):

* [QSA glossary] keieiax.jp, "Qwen Sparse Attention（キューウェン・スパース・
  アテンション）とは" -- section 4トークンずつまとめて、必要な場所を探す: the context
  is first compressed into 4-token micro-blocks, a lightweight learned indexer
  estimates each block's importance, and the public setting keeps at most 512
  blocks (2,048 tokens) per query; section 他のスパースアテンションとの違い: the
  indexer may pick blocks far from the current position; section 長文AIのコ
  ストと応答時間にどう影響する？: the comparison is against dense
  grouped-query attention (GQA).
* [PR #30965 digest] blog.cecily.jp/6295, the paragraph on Raschka's
  explanation: the indexer averages the keys of each block and scores the
  block, and blocks are taken in descending score order, up to 512 blocks;
  the paragraph on the trade-offs: a whole 4-token block is read even if one
  token in it matters, and the budget is 2,048 tokens plus the current
  fractional block.
* [kq_mask explainer] ai-manual.ru, "Экономия VRAM в llama.cpp: что даёт
  QSA-выбор без kq_mask", section "QSA-выбор и kq_mask": a mask removes
  future tokens; the selection can be consumed without materialising one.
* [sparse FA explainer] ai-manual.ru, "llama.cpp получил разреженный Flash
  Attention для Qwen4 на CUDA", section "Разреженный Flash Attention и
  обычный": sparse attention is ordinary softmax attention over a subset of
  token pairs.

The pages do not print the indexer formula.  It is fixed here as
    s_b = sum_h w_h * max(0, q_idx[h] . kbar[b])
(learned per-head weights, ReLU, summed over indexer heads); the other open
points are resolved as follows (each is also listed in the design notes):

* pooled key kbar[b] = mean of the 4 indexer keys of block b, rounded to the
  storage dtype (round to nearest, ties to even);
* a query at absolute position t has own block b_own = t // 4; the candidates
  are blocks 0 .. b_own-1; the own block (tokens 4*b_own .. t) is always
  attended and never competes;
* at most k candidates are kept; ties in score go to the lower block id; the
  kept ids are reported in ascending order;
* one selection per query token, shared by all query heads; query head hq
  uses KV head hq // (Hq // Hkv);
* attention is softmax(scale * q . k) over the token set, in float64;
* the block size is a parameter (default 4).  Block size 1 is the
  token-granular selection the pages contrast QSA with ([PR #30965 digest],
  paragraph on Raschka's explanation: DeepSeek Sparse Attention picks single
  tokens where QSA picks 4-token blocks; paragraph on the trade-offs: the
  block index is the coarser one).  The budget stays 2,048 tokens, so
  top_k = 2048 / block; a block of one token pools to its own key.

Parity status: every function below is pinned by tests/test_oracle_pins.py
(closed forms, invariants, brute force and library routines).  Absolute
attention values have no worked example on the pages; they are pinned through
dense equivalence, masked brute force against torch's CPU
scaled_dot_product_attention, and closed-form special cases.
"""

from __future__ import annotations

import numpy as np

# 4-token micro-blocks ([QSA glossary] 4トークンずつまとめて; [PR #30965 digest]).
BLOCK = 4
# At most 512 blocks = 2,048 tokens per query ([QSA glossary] public setting).
TOP_K_BLOCKS = 512
BUDGET_TOKENS = BLOCK * TOP_K_BLOCKS


# --------------------------------------------------------------------------
# storage-type conversions (exact definitions, no library rounding)
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bfloat16 is the upper 16 bits of an IEEE binary32, so widening is a
    16-bit left shift followed by an exact binary32 -> binary64 conversion.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits), nearest-even.

    Returns the rounded values as float64.  For a normal value with
    |x| = m * 2**e (0.5 <= m < 1) the bfloat16 spacing is 2**(e-8); below
    the binary32 normal range (2**-126) the spacing is the subnormal step
    2**-133.  np.rint rounds exact halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)            # |x| < 2**-126 -> subnormal spacing
    spacing = np.ldexp(1.0, e - 8)
    return np.rint(x / spacing) * spacing


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to binary32 (nearest-even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# step 1: pooling ([PR #30965 digest] keys averaged per block;
#                  [QSA glossary] 4-token micro-blocks)
# --------------------------------------------------------------------------

def pool_blocks(kidx: np.ndarray, dtype: str, b_begin: int = 0,
                b_end: int | None = None, block: int = BLOCK) -> np.ndarray:
    """Pooled indexer keys of complete blocks b_begin .. b_end-1.

    kidx: [L, Di] float64 values of one sequence's indexer keys.
    Returns [b_end - b_begin, Di]: the mean of the `block` keys of each
    block, rounded to the storage dtype.  Only complete blocks exist: b_end
    defaults to L // block and may not exceed it.
    """
    kidx = np.asarray(kidx, dtype=np.float64)
    n_complete = kidx.shape[0] // block
    if b_end is None:
        b_end = n_complete
    if not (0 <= b_begin <= b_end <= n_complete):
        raise ValueError("block range outside the complete blocks")
    out = np.empty((b_end - b_begin, kidx.shape[1]), dtype=np.float64)
    for b in range(b_begin, b_end):
        rows = kidx[block * b: block * b + block]
        out[b - b_begin] = rows.sum(axis=0) / block
    return round_to_storage(out, dtype)


# --------------------------------------------------------------------------
# step 2: candidates (causal block limit) and the own (tail) block
# --------------------------------------------------------------------------

def own_block(t: int, block: int = BLOCK) -> int:
    """Block holding position t; it is the 'current fractional part'."""
    return t // block


def n_candidates(t: int, block: int = BLOCK) -> int:
    """Blocks strictly before the own block compete for selection."""
    return own_block(t, block)


# --------------------------------------------------------------------------
# step 3: indexer score (formula fixed by the spec; learned head weights)
# --------------------------------------------------------------------------

def block_scores(kbar: np.ndarray, q_idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """s[b] = sum_h w[h] * max(0, q_idx[h] . kbar[b]) for every row b of kbar.

    kbar [n, Di], q_idx [Hi, Di], w [Hi]; float64 throughout.  Adding +0.0
    at the end turns a -0.0 into +0.0 so that equal scores compare equal.
    """
    kbar = np.asarray(kbar, dtype=np.float64)
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    s = np.zeros(kbar.shape[0], dtype=np.float64)
    for h in range(q_idx.shape[0]):
        dots = kbar @ q_idx[h]
        s += w[h] * np.maximum(dots, 0.0)
    return s + 0.0


# --------------------------------------------------------------------------
# step 4: top-k selection ([QSA glossary]: at most 512 blocks, best first)
# --------------------------------------------------------------------------

def select_blocks(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Ids of the top_k highest scores (ties -> lower id), ascending.

    Full sort by the key (-score, id); keep the first min(top_k, n); report
    the kept ids in ascending order.
    """
    scores = np.asarray(scores, dtype=np.float64)
    ids = np.arange(scores.shape[0])
    order = np.lexsort((ids, -scores))          # primary -score, then id
    keep = order[: min(top_k, scores.shape[0])]
    return np.sort(keep).astype(np.int64)


# --------------------------------------------------------------------------
# step 5: the token set attended by one query
# --------------------------------------------------------------------------

def token_set(sel: np.ndarray, t: int, block: int = BLOCK) -> np.ndarray:
    """Tokens of the selected blocks, then the own block up to t, ascending."""
    toks = [block * int(b) + i for b in sel for i in range(block)]
    toks += list(range(block * own_block(t, block), t + 1))
    return np.asarray(toks, dtype=np.int64)


def token_set_shared(sel: np.ndarray, t_sel: int, t: int,
                     block: int = BLOCK) -> np.ndarray:
    """Tokens attended at position t >= t_sel by a query that reuses the
    selection made for the query at t_sel (multi-token prediction reusing
    the top index across speculative steps: [QSA glossary], FAQ on whether
    the selection is shared across layers).

    Reading: the reused selection stands for the context before t_sel's own
    block; every token from the start of that block up to t is attended
    (the tail grows with the drafted tokens).  For t == t_sel this is
    token_set(sel, t).
    """
    toks = [block * int(b) + i for b in sel for i in range(block)]
    toks += list(range(block * own_block(t_sel, block), t + 1))
    return np.asarray(toks, dtype=np.int64)


# --------------------------------------------------------------------------
# before step 1: the indexer's input projections
# --------------------------------------------------------------------------

def index_project(x: np.ndarray, wq: np.ndarray, wk: np.ndarray, ww: np.ndarray,
                  n_heads: int, dtype: str):
    """The learned indexer's inputs from hidden states ([QSA glossary],
    section 4トークンずつまとめて: the indexer is learned and light; the pages
    print no projection, so these are plain linear maps).

    x [T, H]; wq [Hi*Di, H], wk [Di, H], ww [Hi, H] (one row per output).
    Returns q_idx [T, Hi, Di] and kidx [T, Di] rounded to the storage dtype,
    and w [T, Hi] rounded to float32.  Each output is the dot product of the
    token's hidden state with one weight row (a matrix product, computed in
    float64).
    """
    x = np.asarray(x, dtype=np.float64)
    q = round_to_storage(x @ np.asarray(wq, dtype=np.float64).T, dtype)
    k = round_to_storage(x @ np.asarray(wk, dtype=np.float64).T, dtype)
    w = round_to_f32(x @ np.asarray(ww, dtype=np.float64).T)
    return q.reshape(x.shape[0], n_heads, -1), k, w


# --------------------------------------------------------------------------
# step 6: attention over the token set
# --------------------------------------------------------------------------

def kv_head_of(hq: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Consecutive query heads share a KV head (grouped-query attention)."""
    return hq // (n_q_heads // n_kv_heads)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, tokens: np.ndarray,
           scale: float) -> np.ndarray:
    """Softmax attention of one query row over the given tokens.

    q [Hq, D]; k, v [L, Hkv, D]; tokens: ids into L.  For each query head,
    z_j = scale * q . k_j, p = exp(z - max z) / sum, out = sum_j p_j v_j.
    """
    q = np.asarray(q, dtype=np.float64)
    hq_n, d = q.shape
    hkv_n = k.shape[1]
    out = np.empty((hq_n, d), dtype=np.float64)
    for hq in range(hq_n):
        hk = kv_head_of(hq, hq_n, hkv_n)
        kk = np.asarray(k[tokens, hk], dtype=np.float64)
        vv = np.asarray(v[tokens, hk], dtype=np.float64)
        z = scale * (kk @ q[hq])
        p = np.exp(z - z.max())
        p /= p.sum()
        out[hq] = p @ vv
    return out


# --------------------------------------------------------------------------
# one query row end to end
# --------------------------------------------------------------------------

def qsa_select_row(kbar: np.ndarray, q_idx: np.ndarray, w: np.ndarray, t: int,
                   top_k: int, block: int = BLOCK) -> np.ndarray:
    """Selected block ids of the query at position t (steps 2-4)."""
    n = n_candidates(t, block)
    s = block_scores(kbar[:n], q_idx, w)
    return select_blocks(s, top_k)


def qsa_row(k: np.ndarray, v: np.ndarray, kbar: np.ndarray, q: np.ndarray,
            q_idx: np.ndarray, w: np.ndarray, t: int, top_k: int,
            scale: float, block: int = BLOCK) -> tuple[np.ndarray, np.ndarray]:
    """(selected ids, attention output [Hq, D]) of the query at position t.

    k, v: [L, Hkv, D] with L > t (the query's own K/V are in the cache);
    kbar: the pooled keys of at least the blocks before the own block.
    """
    sel = qsa_select_row(kbar, q_idx, w, t, top_k, block)
    out = attend(q, k, v, token_set(sel, t, block), scale)
    return sel, out


# --------------------------------------------------------------------------
# side checks: dense causal GQA and masked brute force (matrix form)
# --------------------------------------------------------------------------

def dense_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 pos: np.ndarray, scale: float) -> np.ndarray:
    """Dense causal GQA attention in matrix form (the comparison baseline).

    q [T, Hq, D], k/v [L, Hkv, D], pos [T]: row i sees tokens 0..pos[i].
    """
    mask = np.arange(k.shape[0])[None, :] <= np.asarray(pos)[:, None]
    return masked_attention(q, k, v, mask, scale)


def qsa_mask(sels: list, pos: np.ndarray, n_keys: int, block: int = BLOCK) -> np.ndarray:
    """The boolean [T, L] table a materialised kq_mask would hold.

    Row i allows token j iff block(j) is selected for row i, or j lies in
    row i's own block at or before pos[i].  Only this oracle builds it.
    """
    pos = np.asarray(pos)
    m = np.zeros((len(sels), n_keys), dtype=bool)
    j = np.arange(n_keys)
    for i, sel in enumerate(sels):
        m[i] = np.isin(j // block, np.asarray(sel))
        m[i] |= (j >= block * own_block(int(pos[i]), block)) & (j <= pos[i])
    return m


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     mask: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * Q K^T + log mask) V for every head, matrix form."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    t_n, hq_n, d = q.shape
    hkv_n = k.shape[1]
    out = np.empty((t_n, hq_n, d), dtype=np.float64)
    for hq in range(hq_n):
        hk = kv_head_of(hq, hq_n, hkv_n)
        z = scale * (q[:, hq, :] @ k[:, hk, :].T)          # [T, L]
        z = np.where(mask, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[:, hq, :] = p @ v[:, hk, :]
    return out
