"""GPU parity at block sizes other than QSA's 4: block size 1 is the
token-granular selection the pages contrast QSA with (with the same
2,048-token budget, top_k = 2048), 2, 8 and 16 lie around it.

Pooled keys and selections are compared bit for bit with the oracle;
attention outputs within max-abs 2e-2 (bfloat16) / 1e-4 (float32).
"""

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_32_amd import binding as B
from block_sparse_attention_32_amd import workloads as W

from gpu_helpers import TOL, Problem, assert_sel_row, f64, sel_rows

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS
BLOCKS = [1, 2, 8, 16]


def _say(msg):
    print(msg, flush=True)


def _wl(block, **kw):
    """Rows of one long sequence (permuted pages) at block size `block`,
    budget 2,048 tokens."""
    base = dict(name=f"mixb{block}", n_ctx=131080, n_new=1, n_needles=6, permute_pages=True,
                seed=78, block=block, top_k=O.BUDGET_TOKENS // block)
    base.update(kw)
    return WL["prefill_8k_at_128k"].replace(**base)


# candidate counts at block size 1 (t candidates): none, fewer than top_k,
# one pass (<= 8,192), chunked rows whose union of per-wave tops is smaller
# than top_k, larger, and long rows
POS = [0, 3, 2047, 2048, 2049, 5000, 8192, 8193, 20000, 40001, 70002, 131072]


@pytest.mark.parametrize("block", BLOCKS)
def test_pool_block_sizes_bit_exact(gpu, block):
    _say(f"pool block={block}")
    wl = WL["decode_8x32k"].replace(n_ctx=3000, n_seqs=3, block=block)
    pb = Problem(wl, gpu)
    pb.pool_all()
    torch.cuda.synchronize()
    for s in range(wl.n_seqs):
        assert np.array_equal(pb.gpu_kbar(s), pb.kbar_oracle(s)), f"seq {s}"


def _e2e(pb):
    st = pb.step()
    torch.cuda.synchronize()
    _, sel, n = sel_rows(st.sel, st.n_sel)
    got = f64(st.out)
    worst = 0.0
    for i in range(len(pb.pos_list)):
        want = pb.oracle_select(i)
        assert_sel_row(sel[i], int(n[i]), want, pb.wl.top_k)
        err = np.abs(got[i] - pb.oracle_attend(i, want)).max()
        worst = max(worst, err)
        assert err <= TOL[pb.wl.dtype], f"row {i} t={pb.pos_list[i]} err={err}"
    assert not np.isnan(got).any()
    return st, worst


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("block", BLOCKS)
def test_e2e_block_sizes(gpu, block, mode):
    """Selection (bit-exact) and attention end to end.  decode: few rows
    (chunked top-k, split-K attention); prefill: 72 rows (matrix-core
    indexer, one workgroup per row)."""
    _say(f"e2e block={block} {mode}")
    wl = _wl(block, mode=mode)
    pos = POS if mode == "decode" else sorted(POS * 6)
    pb = Problem(wl, gpu, [0] * len(pos), pos)
    pb.pool_all()
    _, worst = _e2e(pb)
    _say(f"  max err {worst:.3g}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
@pytest.mark.parametrize("block", [1, 2, 16])
def test_e2e_block_sizes_f32(gpu, block, mode):
    """float32 caches take the generic attention kernel and the chunked
    top-k (tiles hold whole blocks)."""
    _say(f"e2e f32 block={block} {mode}")
    wl = WL["tiny_decode"].replace(n_ctx=600, block=block, top_k=64 // block, mode=mode)
    pos = [0, 5, 63, 64, 65, 200, 599, 600]
    pb = Problem(wl, gpu, [0] * len(pos), pos)
    pb.pool_all()
    _e2e(pb)


@pytest.mark.parametrize("block", [1, 16])
def test_attention_decode_shared_block_sizes(gpu, block):
    """Draft rows reusing one selection: the bridge between the selection
    row's own block and a draft row's position spans up to 60 blocks of
    one token."""
    _say(f"attention shared selection block={block}")
    groups = [(2047, [0, 1, 2, 3]), (32766, [0, 2, 4, 9]), (40000, [0, 60]),
              (40003, [0, 57, 60])]
    pos, sel_of = [], []
    for t_s, lags in groups:
        first = len(pos)
        for lag in lags:
            pos.append(t_s + lag)
            sel_of.append(first)
    wl = _wl(block, n_ctx=40100)
    pb = Problem(wl, gpu, [0] * len(pos), pos)
    T = len(pos)
    sel = torch.full((T, wl.top_k), -1, dtype=torch.int32)
    n_sel = torch.full((T,), wl.top_k, dtype=torch.int32)
    sels = {}
    for i in range(T):
        if sel_of[i] == i:
            s_ = pb.oracle_select(i)
            sels[i] = s_
            sel[i, : len(s_)] = torch.from_numpy(s_.astype(np.int32))
            n_sel[i] = len(s_)
        else:
            sel[i] = torch.arange(wl.top_k, dtype=torch.int32)  # must not be used
    out = torch.full_like(pb.qs.q, float("nan"))
    ws = B.workspace(B.QSA_OP_ATTN_DECODE_SHARED, pb.cv, pb.rows, wl.hq, wl.top_k)
    B.qsa_attn_decode_shared(pb.cv, pb.rows, pb.qs.q, sel.to(gpu), n_sel.to(gpu),
                             torch.tensor(sel_of, dtype=torch.int32, device=gpu), wl.top_k,
                             wl.scale, out, ws)
    torch.cuda.synchronize()
    got = f64(out)
    for i in range(T):
        s_ = sel_of[i]
        toks = O.token_set_shared(sels[s_], pos[s_], pos[i], block)
        k, v = pb.token_kv(0, toks)
        want = O.attend(f64(pb.qs.q[i]), k, v, np.arange(len(toks)), wl.scale)
        err = np.abs(got[i] - want).max()
        assert err <= TOL[wl.dtype], f"row {i} t={pos[i]} (selection at {pos[s_]}) err={err}"


@pytest.mark.parametrize("name", ["decode_8x32k_tok", "decode_1m_tok"])
def test_e2e_token_granular_workload(gpu, name):
    """The token-granular benchmark workload itself: every token of every
    planted needle span is selected."""
    _say(f"e2e {name}")
    pb = Problem(WL[name], gpu)
    pb.pool_all()
    st, worst = _e2e(pb)
    _say(f"  max err {worst:.3g}")
    _, sel, n = sel_rows(st.sel, st.n_sel)
    for i, s in enumerate(pb.seq_id_list):
        toks = {4 * b + j for b in pb.cache.needles[s] for j in range(4)}
        assert toks <= set(sel[i, : n[i]].tolist())
