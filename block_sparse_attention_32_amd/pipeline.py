"""One pass of the QSA hot path over a batch of query rows.

Orchestration only: allocates the output and workspace buffers with torch
and calls the libqsa entry points in order (pool the newly completed
blocks, select the top-k blocks per row, attend).  All arithmetic happens
in the HIP kernels.
"""

from __future__ import annotations

import torch

from . import binding as B


class QsaStep:
    """Buffers and calls of one step.

    cache: binding.CacheView; rows: binding.QueriesView; q [T, Hq, D];
    q_idx [T, Hi, Di]; w [T, Hi] float32.  mode "decode" uses the split
    attention kernel, "prefill" one workgroup per row.
    """

    def __init__(self, cache: B.CacheView, rows: B.QueriesView, q, q_idx, w, top_k: int,
                 scale: float, mode: str = "decode"):
        self.cache, self.rows = cache, rows
        self.q, self.q_idx, self.w = q, q_idx, w
        self.top_k, self.scale, self.mode = int(top_k), float(scale), mode
        dev = cache.device
        t = rows.n_rows
        self.sel = torch.empty((t, self.top_k), dtype=torch.int32, device=dev)
        self.n_sel = torch.empty((t,), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q)
        self.ws_topk = B.workspace(B.QSA_OP_TOPK, cache, rows, 0, self.top_k)
        op = B.QSA_OP_ATTN_DECODE if mode == "decode" else B.QSA_OP_ATTN_PREFILL
        self.ws_attn = B.workspace(op, cache, rows, q.shape[1], self.top_k)

    def pool(self, blk_begin: torch.Tensor, max_new_blocks: int):
        B.qsa_pool_blocks(self.cache, blk_begin, max_new_blocks)

    def select(self, scores=None):
        B.qsa_topk_blocks(self.cache, self.rows, self.top_k, self.sel, self.n_sel, self.ws_topk,
                          scores=scores, q_idx=self.q_idx, w=self.w)

    def select_pooling_newest(self):
        """The decode step's pooling and selection in one call: each row's
        newest complete block is pooled, then the rows select (fused)."""
        B.qsa_topk_blocks_pool_newest(self.cache, self.rows, self.top_k, self.sel, self.n_sel,
                                      self.ws_topk, self.q_idx, self.w)

    def attend(self):
        fn = B.qsa_attn_decode if self.mode == "decode" else B.qsa_attn_prefill
        fn(self.cache, self.rows, self.q, self.sel, self.n_sel, self.top_k, self.scale,
           self.out, self.ws_attn)

    def run(self, blk_begin=None, max_new_blocks: int = 0):
        if blk_begin is not None and max_new_blocks > 0:
            self.pool(blk_begin, max_new_blocks)
        self.select()
        self.attend()
        return self.sel, self.n_sel, self.out


class MtpStep:
    """A multi-token decode step (draft tokens of speculative decoding): the
    selection is made for rows 0 .. n_sel_rows - 1 only (each sequence's
    first draft row) and every row attends the selection of row sel_of[i]
    plus its own recent tokens (qsa_attn_decode_shared)."""

    def __init__(self, cache: B.CacheView, rows: B.QueriesView, q, q_idx, w, sel_of,
                 n_sel_rows: int, top_k: int, scale: float):
        self.cache, self.rows, self.q = cache, rows, q
        self.top_k, self.scale, self.n = int(top_k), float(scale), int(n_sel_rows)
        dev = cache.device
        t = rows.n_rows
        n = self.n
        self.sel_of = sel_of
        self.q_idx, self.w = q_idx[:n], w[:n]
        self.sel = torch.full((t, self.top_k), -1, dtype=torch.int32, device=dev)
        self.n_sel = torch.zeros((t,), dtype=torch.int32, device=dev)
        seq_id, pos = rows.tensors
        self.sel_rows = B.QueriesView(seq_id[:n], pos[:n], rows.s.max_pos)
        self.out = torch.empty_like(q)
        self.ws_topk = B.workspace(B.QSA_OP_TOPK, cache, self.sel_rows, 0, self.top_k)
        self.ws_attn = B.workspace(B.QSA_OP_ATTN_DECODE_SHARED, cache, rows, q.shape[1],
                                   self.top_k)

    def select(self):
        B.qsa_topk_blocks(self.cache, self.sel_rows, self.top_k, self.sel[: self.n],
                          self.n_sel[: self.n], self.ws_topk, q_idx=self.q_idx, w=self.w)

    def attend(self):
        B.qsa_attn_decode_shared(self.cache, self.rows, self.q, self.sel, self.n_sel,
                                 self.sel_of, self.top_k, self.scale, self.out, self.ws_attn)


class DenseStep:
    """Dense causal GQA attention of the same rows (comparison baseline)."""

    def __init__(self, cache: B.CacheView, rows: B.QueriesView, q, scale: float,
                 mode: str = "decode"):
        self.cache, self.rows, self.q, self.scale, self.mode = cache, rows, q, float(scale), mode
        self.out = torch.empty_like(q)
        op = B.QSA_OP_DENSE_DECODE if mode == "decode" else B.QSA_OP_DENSE_PREFILL
        self.ws = B.workspace(op, cache, rows, q.shape[1], 0)

    def run(self):
        fn = B.qsa_dense_attn_decode if self.mode == "decode" else B.qsa_dense_attn_prefill
        fn(self.cache, self.rows, self.q, self.scale, self.out, self.ws)
        return self.out


def pool_all(cache: B.CacheView, n_seqs: int, n_blocks: int, device) -> None:
    """Pool blocks 0 .. n_blocks-1 of every sequence (cache set-up)."""
    begin = torch.zeros(n_seqs, dtype=torch.int32, device=device)
    B.qsa_pool_blocks(cache, begin, n_blocks)


class ChunkedPrefill:
    """A prefill in chunks of query rows, chunk by chunk in order.

    chunks: list of (QsaStep, blk_begin, n_new_blocks): the chunk's rows and
    the blocks its tokens complete (pooled before its selection).

    With overlap=True the selections run on the caller's stream and the
    attention calls on a second stream: the attention of chunk c waits
    (HIP event) for the selection of chunk c only, so it runs while the
    selection of chunk c+1 computes.  The two phases stress different units
    (the indexer matrix cores and VALU, the attention the vector-memory
    path), and nothing either writes is read by the other.  Results are the
    same as with overlap=False; the caller's stream waits for the last
    attention before returning.
    """

    def __init__(self, cache: B.CacheView, chunks, overlap: bool = True):
        self.cache, self.chunks, self.overlap = cache, list(chunks), overlap
        self.side = torch.cuda.Stream(device=cache.device) if overlap else None

    def run(self, call=None):
        """call(name, fn, *args): optional wrapper around each library call
        (timing); it runs on the stream current at the call."""
        call = call or (lambda name, fn, *a: fn(*a))
        main = torch.cuda.current_stream()
        for st, begin, nb in self.chunks:
            call("pool", B.qsa_pool_blocks, self.cache, begin, nb)
            call("topk", st.select)
            if not self.overlap:
                call("attn", st.attend)
                continue
            done = torch.cuda.Event()
            done.record(main)
            with torch.cuda.stream(self.side):
                self.side.wait_event(done)
                call("attn", st.attend)
        if self.overlap:
            main.wait_stream(self.side)
