"""Pins of the CPU oracle against closed forms, brute force, invariants and
library routines (CPU only).

Each oracle function is checked by something other than itself, chosen so
that a dropped term, a wrong sign, a wrong index or a transposed operand in
it fails at least one test here.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qsa_constants.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                name, value = line.split()
                vals[name] = int(value)
    return vals


# ---------------------------------------------------------------- constants

def test_constants_match_pages():
    g = _golden()
    assert O.BLOCK == g["block_tokens"]
    assert O.TOP_K_BLOCKS == g["max_blocks"]
    assert O.BLOCK * O.TOP_K_BLOCKS == g["max_tokens_selected"]
    assert g["max_tokens_selected"] + O.BLOCK == g["max_tokens_attended"]


@pytest.mark.parametrize("t", [0, 1, 3, 4, 7, 2047, 2048, 2051, 2052, 5000, 123457])
def test_budget_counts(t):
    """n_sel = min(512, t // 4) and the attended count never exceeds 2,052."""
    g = _golden()
    n_cand = O.n_candidates(t)
    assert n_cand == t // 4
    sel = O.select_blocks(np.zeros(n_cand), O.TOP_K_BLOCKS)
    assert len(sel) == min(g["max_blocks"], t // 4)
    toks = O.token_set(sel, t)
    assert len(toks) == 4 * len(sel) + t % 4 + 1
    assert len(toks) <= g["max_tokens_attended"]
    assert toks.max() == t and len(np.unique(toks)) == len(toks)


# ---------------------------------------------------------------- dtypes

def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    ref = t.to(torch.float64).numpy()
    got = O.bf16_bits_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])


def test_bf16_rounding_closed_forms():
    cases = {
        1.0 + 2.0 ** -8: 1.0,                     # exact half -> even (down)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,     # exact half -> even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,   # above half -> up
        -(1.0 + 2.0 ** -8): -1.0,
        3.0: 3.0,
        2.0 ** -130: 2.0 ** -130,                 # subnormal, representable
        2.0 ** -134: 0.0,                         # half of smallest -> even 0
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.round_to_bf16(np.array([x]))[0] == want, x


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-6, 6, 50000)).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_f32_rounding_closed_forms():
    """binary32 keeps 24 significant bits: the spacing above 1 is 2**-23 and
    the smallest subnormal is 2**-149; exact halves go to the even neighbour."""
    cases = {
        1.0 + 2.0 ** -24: 1.0,                          # half -> even (down)
        1.0 + 3 * 2.0 ** -24: 1.0 + 2.0 ** -22,         # half -> even (up)
        1.0 + 2.0 ** -24 + 2.0 ** -40: 1.0 + 2.0 ** -23,  # above half -> up
        1.0 + 2.0 ** -24 - 2.0 ** -40: 1.0,             # below half -> down
        -(1.0 + 3 * 2.0 ** -24): -(1.0 + 2.0 ** -22),
        2.0 ** -150: 0.0,                               # half the smallest subnormal -> 0
        3 * 2.0 ** -150: 2.0 ** -148,                   # subnormal half -> even (up)
        5 * 2.0 ** -150: 2.0 ** -148,                   # subnormal half -> even (down)
        0.1: 13421773 * 2.0 ** -27,                     # the float32 nearest 0.1
        3.0: 3.0,
    }
    for x, want in cases.items():
        assert O.round_to_f32(np.array([x]))[0] == want, x


def test_pool_f32_mean_rounds_to_nearest_even():
    # rows 1, 1, 1, 1 + 2**-22: the exact mean 1 + 2**-24 lies halfway between
    # the float32 neighbours 1 and 1 + 2**-23 and rounds to the even one, 1
    kidx = np.array([[1.0], [1.0], [1.0], [1.0 + 2.0 ** -22]])
    assert O.pool_blocks(kidx, "f32")[0, 0] == 1.0
    # rows 1, 1, 1, 1 + 3 * 2**-22: mean 1 + 3 * 2**-24 -> 1 + 2**-22
    kidx[3, 0] = 1.0 + 3 * 2.0 ** -22
    assert O.pool_blocks(kidx, "f32")[0, 0] == 1.0 + 2.0 ** -22


# ---------------------------------------------------------------- pooling

def test_pool_closed_forms():
    kidx = np.array([[0.0, 1.0], [0.0, 2.0], [0.0, 3.0], [4.0, 4.0],   # block 0
                     [5.0, -1.0], [5.0, -1.0], [5.0, -1.0], [5.0, -1.0],  # block 1
                     [9.0, 9.0]])                                      # incomplete
    got = O.pool_blocks(kidx, "f32")
    assert got.shape == (2, 2)                  # the incomplete block is not pooled
    assert np.array_equal(got, [[1.0, 2.5], [5.0, -1.0]])
    assert np.array_equal(O.pool_blocks(kidx, "f32", 1, 2), [[5.0, -1.0]])
    with pytest.raises(ValueError):
        O.pool_blocks(kidx, "f32", 0, 3)


def test_pool_rounds_to_storage():
    # mean = 1 + 2**-9: representable in float32, rounds to 1.0 in bfloat16
    kidx = np.array([[1.0], [1.0], [1.0], [1.0 + 2.0 ** -7]])
    assert O.pool_blocks(kidx, "f32")[0, 0] == 1.0 + 2.0 ** -9
    assert O.pool_blocks(kidx, "bf16")[0, 0] == 1.0


def test_pool_homogeneous_and_permutation_invariant():
    rng = np.random.default_rng(2)
    kidx = np.round(rng.standard_normal((64, 16)) * 8) / 8
    a = O.pool_blocks(kidx, "f32")
    assert np.array_equal(O.pool_blocks(2 * kidx, "f32"), 2 * a)
    perm = kidx.reshape(16, 4, 16)[:, ::-1].reshape(64, 16)
    assert np.array_equal(O.pool_blocks(perm, "f32"), a)


# ---------------------------------------------------------------- scoring

def test_scores_select_one_head_and_one_dim():
    rng = np.random.default_rng(3)
    kbar = rng.standard_normal((50, 8))
    for h, d in itertools.product(range(3), range(8)):
        q_idx = np.zeros((3, 8))
        q_idx[h, d] = 1.0
        w = np.zeros(3)
        w[h] = 1.0
        assert np.array_equal(O.block_scores(kbar, q_idx, w), np.maximum(kbar[:, d], 0.0))


def test_scores_closed_form_constant_rows():
    # kbar row b = c_b * ones(Di); q_idx head h = a_h * ones(Di)
    # => dot = Di * c_b * a_h, score = sum_h w_h * max(0, Di * c_b * a_h)
    di = 6
    c = np.array([1.0, -2.0, 0.5, 0.0])
    a = np.array([2.0, -1.0, 3.0])
    w = np.array([0.25, 0.5, 1.0])
    kbar = c[:, None] * np.ones((1, di))
    q_idx = a[:, None] * np.ones((1, di))
    want = [
        0.25 * 12 + 0 + 1.0 * 18,        # c=1:   dots 12, -6, 18
        0 + 0.5 * 12 + 0,                # c=-2:  dots -24, 12, -36
        0.25 * 6 + 0 + 1.0 * 9,          # c=0.5: dots 6, -3, 9
        0.0,
    ]
    assert np.array_equal(O.block_scores(kbar, q_idx, w), want)


def test_scores_invariants():
    rng = np.random.default_rng(4)
    kbar = np.round(rng.standard_normal((40, 16)) * 32) / 32
    q_idx = np.round(rng.standard_normal((4, 16)) * 8) / 8
    w = rng.integers(1, 17, 4) / 16
    s = O.block_scores(kbar, q_idx, w)
    assert np.all(s >= 0)
    # homogeneous in each block's key: scaling block 5 by 3 scales its score by 3
    k2 = kbar.copy()
    k2[5] *= 3
    s2 = O.block_scores(k2, q_idx, w)
    assert s2[5] == 3 * s[5] and np.array_equal(np.delete(s2, 5), np.delete(s, 5))
    # linear in the head weights
    assert np.allclose(O.block_scores(kbar, q_idx, 2 * w), 2 * s, rtol=0, atol=0)
    # heads are interchangeable
    p = [2, 0, 3, 1]
    assert np.allclose(O.block_scores(kbar, q_idx[p], w[p]), s, rtol=1e-15, atol=0)
    # a block anti-aligned with every head scores exactly +0.0
    k3 = kbar.copy()
    k3[7] = -np.sign(q_idx.sum(0))
    q_pos = np.abs(q_idx) * np.sign(q_idx.sum(0))
    s3 = O.block_scores(k3, q_pos, w)
    assert s3[7] == 0.0 and math.copysign(1.0, s3[7]) == 1.0


# ---------------------------------------------------------------- selection

def _brute_force_select(s, k):
    """b is kept iff fewer than k candidates beat it under (score desc, id asc)."""
    n = len(s)
    keep = []
    for b in range(n):
        beaten_by = sum(1 for c in range(n) if s[c] > s[b] or (s[c] == s[b] and c < b))
        if beaten_by < k:
            keep.append(b)
    return keep


def test_select_hand_examples():
    assert O.select_blocks(np.array([3, 1, 4, 1, 5, 9, 2, 6.0]), 3).tolist() == [4, 5, 7]
    assert O.select_blocks(np.array([2, 5, 5, 1.0]), 2).tolist() == [1, 2]
    assert O.select_blocks(np.array([5, 2, 5, 5.0]), 2).tolist() == [0, 2]
    assert O.select_blocks(np.array([1.0, 2.0]), 4).tolist() == [0, 1]
    assert O.select_blocks(np.zeros(0), 4).tolist() == []
    assert O.select_blocks(np.zeros(700), 512).tolist() == list(range(512))


@pytest.mark.parametrize("seed", range(8))
def test_select_matches_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    n = int(rng.integers(1, 120))
    k = int(rng.integers(1, 40))
    s = rng.integers(0, 12, n).astype(np.float64) / 4   # many ties
    assert O.select_blocks(s, k).tolist() == _brute_force_select(s, k)


# ---------------------------------------------------------------- token set

def test_token_set_closed_form():
    assert O.token_set(np.array([0, 2]), 13).tolist() == [0, 1, 2, 3, 8, 9, 10, 11, 12, 13]
    assert O.token_set(np.array([], dtype=np.int64), 0).tolist() == [0]
    # a full own block (t = 4b+3) is attended as the tail, not as a candidate
    assert O.token_set(np.array([1]), 11).tolist() == [4, 5, 6, 7, 8, 9, 10, 11]


def test_token_set_shared_closed_form():
    """A query reusing the selection made 4 positions earlier: the reused
    blocks, then everything from the earlier query's own block on."""
    assert O.token_set_shared(np.array([0, 2]), 13, 17).tolist() == \
        [0, 1, 2, 3, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17]
    assert O.token_set_shared(np.array([], dtype=np.int64), 3, 5).tolist() == [0, 1, 2, 3, 4, 5]
    # the drafted tokens cross into the next block: 8..9 join the tail
    assert O.token_set_shared(np.array([0]), 6, 9).tolist() == list(range(10))


@pytest.mark.parametrize("t_sel", [0, 5, 13, 40])
def test_token_set_shared_reduces_to_token_set(t_sel):
    rng = np.random.default_rng(t_sel)
    n = t_sel // 4
    sel = np.sort(rng.choice(n, size=min(n, 3), replace=False)) if n else np.array([], np.int64)
    assert O.token_set_shared(sel, t_sel, t_sel).tolist() == O.token_set(sel, t_sel).tolist()


@pytest.mark.parametrize("t_sel,t", [(13, 13), (13, 16), (13, 19), (6, 30), (0, 3)])
def test_shared_selection_covering_context_is_dense(t_sel, t):
    """When the reused selection holds every block before t_sel's own block,
    a later draft position attends its whole causal prefix: the result is
    dense causal attention (pinned to torch SDPA above)."""
    rng = np.random.default_rng(t)
    k = rng.standard_normal((t + 1, 2, 8))
    v = rng.standard_normal((t + 1, 2, 8))
    q = rng.standard_normal((4, 8))
    sel = np.arange(t_sel // 4)
    got = O.attend(q, k, v, O.token_set_shared(sel, t_sel, t), 0.3)
    want = O.dense_causal(q[None], k, v, np.array([t]), 0.3)[0]
    assert np.allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- projections

def test_index_project_one_hot_states_read_weight_columns():
    """A one-hot hidden state picks column c of every weight matrix: q_idx,
    kidx and w are those columns (rounded), laid out head by head."""
    rng = np.random.default_rng(11)
    h, hi, di = 12, 3, 4
    wq = rng.integers(-40, 40, (hi * di, h)) / 16.0
    wk = rng.integers(-40, 40, (di, h)) / 16.0
    ww = rng.standard_normal((hi, h))
    x = np.eye(h)[[5, 0, 11]]
    q, k, w = O.index_project(x, wq, wk, ww, hi, "bf16")
    for t, c in enumerate([5, 0, 11]):
        for head in range(hi):
            assert q[t, head].tolist() == wq[head * di:(head + 1) * di, c].tolist()
        assert k[t].tolist() == wk[:, c].tolist()
        assert w[t].tolist() == O.round_to_f32(ww[:, c]).tolist()


def test_index_project_hand_example():
    # x = (1, 2), wq rows (1, 0), (0, 1), (1, 1), (2, -1) -> heads [[1, 2], [3, 0]]
    x = np.array([[1.0, 2.0]])
    wq = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, -1.0]])
    wk = np.array([[0.5, 0.25], [-1.0, 1.0]])
    ww = np.array([[0.1, 0.2]])
    q, k, w = O.index_project(x, wq, wk, ww, 2, "f32")
    assert q.tolist() == [[[1.0, 2.0], [3.0, 0.0]]]
    assert k.tolist() == [[1.0, 1.0]]
    assert w.tolist() == [[float(np.float32(0.5))]]


def test_index_project_rounds_bf16():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    x = np.array([[1.0, 2.0 ** -8]])
    wq = np.array([[1.0, 1.0]])
    q, k, _ = O.index_project(x, wq, wq, wq, 1, "bf16")
    assert q[0, 0, 0] == 1.0 and k[0, 0] == 1.0


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, mask, scale):
    """torch CPU scaled_dot_product_attention in float64 with GQA expansion."""
    t_n, hq, d = q.shape
    hkv = k.shape[1]
    rep = hq // hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))          # [Hq,T,D]
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k, rep, axis=1).transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, rep, axis=1).transpose(1, 0, 2)))
    m = torch.from_numpy(mask)[None].expand(hq, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.numpy().transpose(1, 0, 2)


def test_attend_closed_forms():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((10, 2, 4))
    v = rng.standard_normal((10, 2, 4))
    toks = np.array([1, 4, 6, 7])
    # q = 0: uniform weights -> mean of V over the tokens, per KV head
    out = O.attend(np.zeros((4, 4)), k, v, toks, 0.5)
    for hq in range(4):
        assert np.allclose(out[hq], v[toks, hq // 2].mean(0), atol=1e-15)
    # constant V -> that constant
    vc = np.ones_like(v) * 3.5
    assert np.allclose(O.attend(rng.standard_normal((4, 4)), k, vc, toks, 0.3), 3.5, atol=1e-14)
    # a single token -> its V row
    out1 = O.attend(rng.standard_normal((4, 4)), k, v, np.array([6]), 1.0)
    assert np.array_equal(out1[3], v[6, 1])
    # two tokens: weight of token a = 1 / (1 + exp(z_b - z_a))
    q = rng.standard_normal((2, 4))
    k1 = k[:, :1]
    v1 = v[:, :1]
    za = 0.7 * q[0] @ k1[2, 0]
    zb = 0.7 * q[0] @ k1[5, 0]
    pa = 1.0 / (1.0 + math.exp(zb - za))
    want = pa * v1[2, 0] + (1 - pa) * v1[5, 0]
    assert np.allclose(O.attend(q, k1, v1, np.array([2, 5]), 0.7)[0], want, atol=1e-14)


def test_attend_permutation_invariant():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((30, 2, 8))
    v = rng.standard_normal((30, 2, 8))
    q = rng.standard_normal((4, 8))
    toks = np.array([0, 3, 4, 9, 17, 22, 29])
    a = O.attend(q, k, v, toks, 0.35)
    b = O.attend(q, k, v, toks[::-1].copy(), 0.35)
    assert np.allclose(a, b, rtol=0, atol=1e-14)


def test_dense_causal_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((9, 4, 8))
    k = rng.standard_normal((20, 2, 8))
    v = rng.standard_normal((20, 2, 8))
    pos = np.array([0, 1, 3, 4, 7, 11, 12, 18, 19])
    mask = np.arange(20)[None, :] <= pos[:, None]
    got = O.dense_causal(q, k, v, pos, 0.4)
    assert np.allclose(got, _sdpa(q, k, v, mask, 0.4), rtol=0, atol=1e-12)


def _random_problem(rng, L, hq=4, hkv=2, d=8, hi=2, di=8):
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    kidx = np.round(rng.standard_normal((L, di)) * 8) / 8
    return k, v, kidx


@pytest.mark.parametrize("seed", range(4))
def test_masked_bruteforce_matches_rows_and_torch(seed):
    """PIN-6: per-row attention over the token set equals matrix-form
    softmax(QK^T*scale + log M)V under the explicit block mask, and torch's
    masked scaled_dot_product_attention."""
    rng = np.random.default_rng(20 + seed)
    L = int(rng.integers(12, 90))
    k, v, kidx = _random_problem(rng, L)
    kbar = O.pool_blocks(kidx, "f32")
    top_k = int(rng.integers(1, 6))
    pos = np.sort(rng.choice(L, size=min(L, 7), replace=False))
    q = rng.standard_normal((len(pos), 4, 8))
    q_idx = np.round(rng.standard_normal((len(pos), 2, 8)) * 8) / 8
    w = rng.integers(1, 17, (len(pos), 2)) / 16
    sels, rows = [], []
    for i, t in enumerate(pos):
        sel, out = O.qsa_row(k, v, kbar, q[i], q_idx[i], w[i], int(t), top_k, 0.3)
        sels.append(sel)
        rows.append(out)
    mask = O.qsa_mask(sels, pos, L)
    for i, t in enumerate(pos):
        assert mask[i].sum() == 4 * len(sels[i]) + int(t) % 4 + 1
        assert not mask[i, int(t) + 1:].any()              # causal
    mat = O.masked_attention(q, k, v, mask, 0.3)
    assert np.allclose(np.stack(rows), mat, rtol=0, atol=1e-12)
    assert np.allclose(mat, _sdpa(q, k, v, mask, 0.3), rtol=0, atol=1e-12)


def test_dense_equivalence_when_budget_covers_context():
    """PIN-5: with t // 4 <= k every earlier block is selected, so QSA equals
    dense causal attention (bit-identical to attend over 0..t)."""
    rng = np.random.default_rng(30)
    L = 65
    k, v, kidx = _random_problem(rng, L, hq=4, hkv=1, d=32, hi=2, di=16)
    kbar = O.pool_blocks(kidx, "f32")
    pos = np.arange(L)
    q = rng.standard_normal((L, 4, 32))
    q_idx = np.round(rng.standard_normal((L, 2, 16)) * 8) / 8
    w = rng.integers(1, 17, (L, 2)) / 16
    dense = O.dense_causal(q, k, v, pos, 32 ** -0.5)
    for i, t in enumerate(pos):
        sel, out = O.qsa_row(k, v, kbar, q[i], q_idx[i], w[i], int(t), 16, 32 ** -0.5)
        assert sel.tolist() == list(range(int(t) // 4))
        full = O.attend(q[i], k, v, np.arange(int(t) + 1), 32 ** -0.5)
        assert np.array_equal(out, full)
        assert np.allclose(out, dense[i], rtol=0, atol=1e-12)


def test_end_to_end_hand_example():
    """Query at t=9 (own block 2 = tokens 8, 9); candidates blocks 0 and 1;
    block 1 has the larger pooled key along the indexer query, so with k=1
    the token set is {4..7, 8, 9}.  With Q = 0 the softmax is uniform and
    the output is the mean of V over those six tokens."""
    L = 12
    kidx = np.zeros((L, 2))
    kidx[4:8, 0] = 1.0                   # block 1: kbar = (1, 0)
    kidx[0:4, 0] = -1.0                  # block 0: kbar = (-1, 0) -> ReLU 0
    kbar = O.pool_blocks(kidx, "f32")
    v = np.arange(L * 1 * 3, dtype=np.float64).reshape(L, 1, 3)
    k = np.ones((L, 1, 3))
    sel, out = O.qsa_row(k, v, kbar, np.zeros((2, 3)), np.array([[1.0, 0.0]]),
                         np.array([1.0]), 9, 1, 1.0)
    assert sel.tolist() == [1]
    want = v[[4, 5, 6, 7, 8, 9], 0].mean(0)
    assert np.allclose(out[0], want, atol=1e-13) and np.allclose(out[1], want, atol=1e-13)


# ---------------------------------------------------------------- block sizes
# Block size 1 is the token-granular (DeepSeek-style) selection the pages
# contrast QSA with; the budget stays 2,048 tokens, so top_k = 2048 / block.

def test_pool_block_sizes_closed_forms():
    kidx = np.arange(32, dtype=np.float64)[:, None] * np.array([[1.0, -2.0]])
    # a block of one token pools to its own key
    assert np.array_equal(O.pool_blocks(kidx, "f32", block=1), kidx)
    # pairs: mean of rows 2b, 2b+1 = (4b + 1) / 2 * (1, -2)
    got2 = O.pool_blocks(kidx, "f32", block=2)
    assert got2.shape == (16, 2)
    assert np.array_equal(got2[:, 0], 2.0 * np.arange(16) + 0.5)
    # blocks of 8 and 16: midpoints of the ramp
    assert np.array_equal(O.pool_blocks(kidx, "f32", block=8)[:, 0], [3.5, 11.5, 19.5, 27.5])
    assert np.array_equal(O.pool_blocks(kidx, "f32", block=16)[:, 1], [-15.0, -47.0])
    # an incomplete trailing block is not pooled
    assert O.pool_blocks(kidx[:31], "f32", block=8).shape == (3, 2)


@pytest.mark.parametrize("block", [1, 2, 8, 16])
@pytest.mark.parametrize("t", [0, 1, 15, 16, 17, 2047, 2048, 4097, 70001])
def test_budget_counts_block_sizes(block, t):
    """n_sel = min(2048 / block, t // block); at most 2,048 tokens are
    selected and the own block adds t % block + 1."""
    top_k = O.BUDGET_TOKENS // block
    n_cand = O.n_candidates(t, block)
    assert n_cand == t // block
    sel = O.select_blocks(np.zeros(n_cand), top_k)
    toks = O.token_set(sel, t, block)
    assert len(toks) == block * min(top_k, t // block) + t % block + 1
    assert len(toks) <= O.BUDGET_TOKENS + block
    assert toks.max() == t and len(np.unique(toks)) == len(toks)


def test_token_set_block_sizes_closed_forms():
    assert O.token_set(np.array([3, 7]), 9, 1).tolist() == [3, 7, 9]
    assert O.token_set(np.array([0, 2]), 7, 2).tolist() == [0, 1, 4, 5, 6, 7]
    assert O.token_set(np.array([1]), 20, 8).tolist() == list(range(8, 21))
    assert O.token_set(np.array([0]), 33, 16).tolist() == list(range(16)) + [32, 33]
    assert O.token_set_shared(np.array([2, 5]), 9, 11, 1).tolist() == [2, 5, 9, 10, 11]
    assert O.token_set_shared(np.array([0]), 17, 18, 8).tolist() == list(range(8)) + [16, 17, 18]


@pytest.mark.parametrize("block", [2, 4, 8, 16])
@pytest.mark.parametrize("seed", range(3))
def test_token_granular_selection_of_blockwise_constant_keys(block, seed):
    """When the indexer keys are constant inside every block and t is a
    block start, the token-granular selection with budget k * block picks
    exactly the tokens of the k blocks the block-level selection picks:
    tokens of one block tie and ties go to the lower id, so whole blocks
    are taken in the block order, and the two own blocks are both {t}."""
    rng = np.random.default_rng(40 + seed)
    n_blocks = int(rng.integers(5, 40))
    t = block * n_blocks
    keys = np.round(rng.standard_normal((n_blocks + 1, 8)) * 4) / 4
    kidx = np.repeat(keys, block, axis=0)               # [t + block, 8]
    q_idx = np.round(rng.standard_normal((3, 8)) * 4) / 4
    w = rng.integers(1, 9, 3) / 8
    k = int(rng.integers(1, n_blocks + 3))
    sel_b = O.qsa_select_row(O.pool_blocks(kidx, "f32", block=block), q_idx, w, t, k, block)
    sel_t = O.qsa_select_row(O.pool_blocks(kidx, "f32", block=1), q_idx, w, t, k * block, 1)
    assert O.token_set(sel_t, t, 1).tolist() == O.token_set(sel_b, t, block).tolist()


@pytest.mark.parametrize("block", [1, 2, 8])
def test_dense_equivalence_block_sizes(block):
    """With t // block <= k every earlier block is selected: dense causal."""
    rng = np.random.default_rng(31 + block)
    L = 40
    k, v, kidx = _random_problem(rng, L, hq=4, hkv=2, d=8, hi=2, di=8)
    kbar = O.pool_blocks(kidx, "f32", block=block)
    q = rng.standard_normal((L, 4, 8))
    q_idx = np.round(rng.standard_normal((L, 2, 8)) * 8) / 8
    w = rng.integers(1, 17, (L, 2)) / 16
    dense = O.dense_causal(q, k, v, np.arange(L), 0.3)
    for t in range(L):
        sel, out = O.qsa_row(k, v, kbar, q[t], q_idx[t], w[t], t, L, 0.3, block)
        assert sel.tolist() == list(range(t // block))
        assert np.allclose(out, dense[t], rtol=0, atol=1e-12)


@pytest.mark.parametrize("block", [1, 2, 16])
def test_masked_bruteforce_block_sizes(block):
    """Per-row attention over the token set equals the masked matrix form
    and torch's masked SDPA at other block sizes too."""
    rng = np.random.default_rng(50 + block)
    L = 70
    k, v, kidx = _random_problem(rng, L)
    kbar = O.pool_blocks(kidx, "f32", block=block)
    pos = np.sort(rng.choice(L, size=6, replace=False))
    q = rng.standard_normal((len(pos), 4, 8))
    q_idx = np.round(rng.standard_normal((len(pos), 2, 8)) * 8) / 8
    w = rng.integers(1, 17, (len(pos), 2)) / 16
    top_k = 3
    sels, rows = [], []
    for i, t in enumerate(pos):
        sel, out = O.qsa_row(k, v, kbar, q[i], q_idx[i], w[i], int(t), top_k, 0.3, block)
        sels.append(sel)
        rows.append(out)
    mask = O.qsa_mask(sels, pos, L, block)
    for i, t in enumerate(pos):
        assert mask[i].sum() == block * len(sels[i]) + int(t) % block + 1
    mat = O.masked_attention(q, k, v, mask, 0.3)
    assert np.allclose(np.stack(rows), mat, rtol=0, atol=1e-12)
    assert np.allclose(mat, _sdpa(q, k, v, mask, 0.3), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- properties

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 80), block=st.sampled_from([1, 2, 4, 8]), top_k=st.integers(1, 12),
       seed=st.integers(0, 2 ** 16))
def test_property_row_equals_masked_matrix_form(L, block, top_k, seed):
    """On random tiny problems (context 1..80, every t mod block): the token
    set is causal, holds the own block's tail and block * n_sel selected
    tokens, and per-row attention equals the masked matrix form."""
    rng = np.random.default_rng(seed)
    k, v, kidx = _random_problem(rng, L)
    kbar = O.pool_blocks(kidx, "f32", block=block)
    t = int(rng.integers(0, L))
    q = rng.standard_normal((1, 4, 8))
    q_idx = np.round(rng.standard_normal((2, 8)) * 8) / 8
    w = rng.integers(1, 17, 2) / 16
    sel, out = O.qsa_row(k, v, kbar, q[0], q_idx, w, t, top_k, 0.3, block)
    assert len(sel) == min(top_k, t // block)
    toks = O.token_set(sel, t, block)
    assert toks.max() == t and len(toks) == block * len(sel) + t % block + 1
    mask = O.qsa_mask([sel], np.array([t]), L, block)
    assert mask.sum() == len(toks) and not mask[0, t + 1:].any()
    assert np.allclose(out[None], O.masked_attention(q, k, v, mask, 0.3), rtol=0, atol=1e-12)
