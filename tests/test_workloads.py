"""Generator checks (CPU): grid exactness, needle planting, page tables,
and the needle margin the workloads promise (checked through the oracle)."""

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_32_amd import workloads as W


def _np(t):
    return t.to(torch.float64).numpy()


def test_workload_table():
    wl = W.WORKLOADS
    assert wl["tiny_decode"].top_k == 4 and wl["tiny_decode"].dtype == "f32"
    for name in ("decode_8x32k", "decode_1m", "prefill_8k_at_128k", "prefill_1m"):
        w = wl[name]
        assert (w.hq, w.hkv, w.d, w.hi, w.di, w.top_k, w.page_size) == (16, 2, 128, 4, 64, 512, 64)
    assert wl["decode_1m"].total_len == 1048577
    assert wl["prefill_1m"].chunk == 32768 and wl["prefill_1m"].n_new == 1 << 20


def test_page_table_is_a_permutation():
    wl = W.WORKLOADS["decode_8x32k"].replace(n_ctx=1000)
    c = W.make_cache(wl)
    bt = c.block_table.flatten().tolist()
    assert sorted(bt) == list(range(c.n_pages))
    assert bt != list(range(c.n_pages))


def test_grid_makes_fp32_indexer_exact():
    """On the grid, float32 pooling and scoring in two different orders equal
    the float64 result exactly (so any GPU summation order is exact)."""
    wl = W.WORKLOADS["decode_8x32k"].replace(n_ctx=4000, n_seqs=1)
    c = W.make_cache(wl)
    _, _, kidx = W.seq_view(c, 0)
    kid = _np(kidx)
    qs = W.make_queries(wl, c, [0], [wl.total_len - 1])
    q_idx = _np(qs.q_idx[0])
    w = qs.w[0].double().numpy()
    kbar64 = O.pool_blocks(kid, "bf16")
    # float32 pooling in order ((k0+k1)+k2)+k3 then * 0.25
    nb = kid.shape[0] // 4
    k32 = kid[: 4 * nb].astype(np.float32).reshape(nb, 4, wl.di)
    p32 = (((k32[:, 0] + k32[:, 1]) + k32[:, 2]) + k32[:, 3]) * np.float32(0.25)
    assert np.array_equal(p32.astype(np.float64), kbar64)
    # float32 dots, forward and reversed accumulation
    kb32 = kbar64.astype(np.float32)
    fwd = np.zeros((kb32.shape[0], wl.hi), np.float32)
    rev = np.zeros_like(fwd)
    for d in range(wl.di):
        fwd += kb32[:, d:d + 1] * q_idx[None, :, d].astype(np.float32)
        rev += kb32[:, wl.di - 1 - d:wl.di - d] * q_idx[None, :, wl.di - 1 - d].astype(np.float32)
    assert np.array_equal(fwd, rev)
    s32 = (np.maximum(fwd, 0) * w.astype(np.float32)).sum(1, dtype=np.float32)
    assert np.array_equal(s32.astype(np.float64), O.block_scores(kbar64, q_idx, w))


@pytest.mark.parametrize("name", ["tiny_decode", "decode_8x32k", "decode_1m"])
def test_needles_selected_with_margin(name):
    """PIN-7: every planted needle is selected, and its score clears the best
    non-needle score by 3 standard deviations of the non-needle scores."""
    wl = W.WORKLOADS[name]
    if name == "decode_1m":
        wl = wl.replace(n_ctx=1 << 17)       # 32,768 candidate blocks on CPU
    if name == "decode_8x32k":
        wl = wl.replace(n_seqs=2)
    c = W.make_cache(wl)
    seq_id, pos = W.decode_rows(wl)
    qs = W.make_queries(wl, c, seq_id, pos)
    for s in range(wl.n_seqs):
        _, _, kidx = W.seq_view(c, s)
        kbar = O.pool_blocks(_np(kidx), wl.dtype)
        t = pos[s]
        n = O.n_candidates(t)
        sc = O.block_scores(kbar[:n], _np(qs.q_idx[s]), qs.w[s].double().numpy())
        needles = c.needles[s]
        assert len(needles) == (len(wl.needle_depths) or wl.n_needles)
        other = np.delete(sc, needles)
        assert sc[needles].min() >= other.max() + 3 * other.std()
        sel = O.select_blocks(sc, wl.top_k)
        assert set(needles) <= set(sel.tolist())


def test_prefill_needles_selected_by_every_later_query():
    wl = W.WORKLOADS["prefill_8k_at_128k"].replace(n_ctx=4096, n_new=256)
    c = W.make_cache(wl)
    seq_id, pos = W.prefill_rows(wl)
    qs = W.make_queries(wl, c, seq_id, pos)
    _, _, kidx = W.seq_view(c, 0)
    kbar = O.pool_blocks(_np(kidx), "bf16")
    for i in range(0, len(pos), 17):
        t = pos[i]
        sel = O.qsa_select_row(kbar, _np(qs.q_idx[i]), qs.w[i].double().numpy(), t, wl.top_k)
        assert set(c.needles[0]) <= set(sel.tolist())


def test_decode_depth_needles():
    wl = W.WORKLOADS["decode_1m"].replace(n_ctx=4000)
    c = W.make_cache(wl)
    n = (wl.total_len - 1) // 4
    assert c.needles[0] == sorted({min(int(d * n), n - 1) for d in wl.needle_depths})
    assert c.needles[0][0] == 0 and c.needles[0][-1] == int(0.99 * n)


def test_generation_is_seeded():
    wl = W.WORKLOADS["tiny_decode"]
    a = W.make_cache(wl)
    b = W.make_cache(wl)
    assert torch.equal(a.k, b.k) and torch.equal(a.kidx, b.kidx)
    assert a.needles == b.needles


@pytest.mark.parametrize("tok,blk", [("prefill_8k_at_128k_tok", "prefill_8k_at_128k"),
                                     ("decode_8x32k_tok", "decode_8x32k"),
                                     ("decode_1m_tok", "decode_1m")])
def test_token_granular_workloads_share_inputs(tok, blk):
    """The token-granular workloads draw the same inputs as the block
    workloads they are named after; only the block size (1) and the budget
    (2,048 tokens, so top_k = 2048) differ."""
    a, b = W.WORKLOADS[tok], W.WORKLOADS[blk]
    assert (a.block, a.top_k) == (1, 2048) and (b.block, b.top_k) == (4, 512)
    assert a.replace(name=b.name, block=4, top_k=512) == b
    small = dict(n_ctx=2048, n_new=4, n_seqs=1)
    ca, cb = W.make_cache(a.replace(**small)), W.make_cache(b.replace(**small))
    assert torch.equal(ca.k, cb.k) and torch.equal(ca.kidx, cb.kidx) and ca.needles == cb.needles
    assert ca.kbar.shape[1] == 4 * cb.kbar.shape[1] == a.page_size


def test_token_granular_selects_needle_tokens():
    """At block size 1 every token of a planted needle span is selected."""
    wl = W.WORKLOADS["decode_8x32k_tok"].replace(n_ctx=12000, n_seqs=1)
    c = W.make_cache(wl)
    seq_id, pos = W.decode_rows(wl)
    qs = W.make_queries(wl, c, seq_id, pos)
    _, _, kidx = W.seq_view(c, 0)
    kbar = O.pool_blocks(_np(kidx), wl.dtype, block=1)
    sel = O.qsa_select_row(kbar, _np(qs.q_idx[0]), qs.w[0].double().numpy(), pos[0],
                           wl.top_k, block=1)
    toks = {4 * b + i for b in c.needles[0] for i in range(4)}
    assert len(sel) == 2048 and toks <= set(sel.tolist())
