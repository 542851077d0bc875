"""Child process of tests/test_gpu_debug.py: runs the same small decode and
prefill calls on whichever libqsa QSA_LIB names, then calls with invalid
device data, and prints one JSON line: the debug bits recorded per case and
the path of the saved valid-case results."""

import json
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_attention_32_amd import binding as B  # noqa: E402
from block_sparse_attention_32_amd import pipeline as P  # noqa: E402
from block_sparse_attention_32_amd import workloads as W  # noqa: E402

WL = W.WORKLOADS["decode_8x32k"].replace(name="dbg", n_ctx=6000, n_seqs=3, n_needles=3,
                                          permute_pages=True, seed=5)


def take(debug):
    return B.qsa_debug_take() if debug else 0


def run_cases(debug, out_path):
    dev = torch.device("cuda:0")
    cache = W.make_cache(WL, device=dev)
    cv = B.CacheView.from_cache(cache)
    P.pool_all(cv, WL.n_seqs, WL.total_len // 4, dev)
    res, flags = {}, {}
    # valid: decode rows (chunked top-k, split attention) and 80 prefill rows
    # of sequence 1 (matrix-core indexer, per-row attention)
    seq_id, pos = W.decode_rows(WL)
    qs = W.make_queries(WL, cache, seq_id, pos, device=dev)
    dec = P.QsaStep(cv, B.QueriesView(qs.seq_id, qs.pos, max(pos)), qs.q, qs.q_idx, qs.w,
                    WL.top_k, WL.scale, "decode")
    dec.select_pooling_newest()
    dec.attend()
    ppos = list(range(2000, 6000, 50))
    pq = W.make_queries(WL, cache, [1] * len(ppos), ppos, device=dev, seed=9)
    pre = P.QsaStep(cv, B.QueriesView(pq.seq_id, pq.pos, max(ppos)), pq.q, pq.q_idx, pq.w,
                    WL.top_k, WL.scale, "prefill")
    pre.run()
    torch.cuda.synchronize()
    flags["valid"] = take(debug)
    res = {k: v.cpu() for k, v in (("dec_sel", dec.sel), ("dec_n", dec.n_sel),
                                   ("dec_out", dec.out), ("pre_sel", pre.sel),
                                   ("pre_n", pre.n_sel), ("pre_out", pre.out),
                                   ("kbar", cache.kbar))}
    torch.save(res, out_path)
    if not debug:
        return flags
    # a page id one past the pool the cache declares: the declared pool is
    # one page short of the allocation, and a table entry names that last
    # page, so the unchecked access would still fall inside the allocation
    n_pages = cache.k.shape[0]
    bt = cache.block_table.clone()
    last = int((bt == n_pages - 1).nonzero()[0, 0]), int((bt == n_pages - 1).nonzero()[0, 1])
    short = B.CacheView(cache.k, cache.v, cache.kidx, cache.kbar, bt, cache.seq_len,
                        WL.total_len)
    short.s.n_pages = n_pages - 1
    st = P.QsaStep(short, B.QueriesView(qs.seq_id, qs.pos, max(pos)), qs.q, qs.q_idx, qs.w,
                   WL.top_k, WL.scale, "decode")
    st.run()
    pst = P.QsaStep(short, B.QueriesView(pq.seq_id, pq.pos, max(ppos)), pq.q, pq.q_idx, pq.w,
                    WL.top_k, WL.scale, "prefill")
    pst.run()
    torch.cuda.synchronize()
    flags["bad_page"] = take(True)
    flags["bad_page_at"] = list(last)
    # a sequence id past n_seqs and a negative position (clamped)
    bad_seq = qs.seq_id.clone()
    bad_seq[0] = WL.n_seqs + 2
    bad_pos = qs.pos.clone()
    bad_pos[1] = -3
    st = P.QsaStep(cv, B.QueriesView(bad_seq, bad_pos, max(pos)), qs.q, qs.q_idx, qs.w,
                   WL.top_k, WL.scale, "decode")
    st.run()
    torch.cuda.synchronize()
    flags["bad_row"] = take(True)
    # a selection length past top_k and a selected id past the row's blocks
    dec.n_sel[0] = WL.top_k + 5
    dec.sel[1, 3] = pos[1] // 4 + 10
    dec.attend()
    torch.cuda.synchronize()
    flags["bad_sel"] = take(True)
    # the same in the many-row (paired) prefill attention: a selected id past
    # the row's blocks in row 3, which shares a workgroup with row 2
    pre.sel[3, 5] = ppos[3] // 4 + 7
    pre.attend()
    torch.cuda.synchronize()
    flags["bad_sel_prefill"] = take(True)
    return flags


if __name__ == "__main__":
    debug = "debug" in os.path.basename(B.LIB_PATH)
    print(f"child: {B.LIB_PATH}", file=sys.stderr, flush=True)
    flags = run_cases(debug, sys.argv[1])
    print(json.dumps(flags), flush=True)
