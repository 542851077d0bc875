"""The C ABI on the host (no GPU work): every declared symbol is exported,
workspace sizing is deterministic, and invalid arguments are rejected
before anything is enqueued."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_32_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "qsa.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(libqsa):
    names = declared()
    assert set(names) == set(B.SYMBOLS)
    for n in names:
        assert hasattr(libqsa, n), n


def test_status_strings(libqsa):
    assert libqsa.qsa_status_string(0) == b"ok"
    for s in (-1, -2, -3, -4):
        assert libqsa.qsa_status_string(s) not in (b"ok", b"unknown status")
    assert libqsa.qsa_version() >= 1


def _cache(**kw):
    d = dict(dtype=1, page_size=64, n_kv_heads=2, head_dim=128, idx_dim=64, n_seqs=2,
             max_pages_per_seq=16, max_seq_len=1000, n_pages=32, block_table=8, seq_len=8,
             k=8, v=8, kidx=8, kbar=8)
    d.update(kw)
    return B._Cache(**d)


def _rows(**kw):
    d = dict(n_rows=3, max_pos=999, seq_id=8, pos=8)
    d.update(kw)
    return B._Queries(**d)


R = ctypes.byref


def test_workspace_sizes(libqsa):
    c, q = _cache(), _rows()
    ws = libqsa.qsa_workspace_size
    assert ws(B.QSA_OP_TOPK, R(c), R(q), 0, 512) > 0
    assert ws(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 512) > 0
    assert ws(B.QSA_OP_ATTN_PREFILL, R(c), R(q), 16, 512) == 0   # one workgroup per row
    assert ws(B.QSA_OP_DENSE_PREFILL, R(c), R(q), 16, 0) == 0
    assert ws(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 512) == ws(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 512)
    # rows reusing a selection also attend the bridge blocks: never less
    assert ws(B.QSA_OP_ATTN_DECODE_SHARED, R(c), R(q), 16, 512) >= ws(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 512)
    assert ws(99, R(c), R(q), 16, 512) == 0
    assert ws(B.QSA_OP_TOPK, None, R(q), 0, 512) == 0
    # bigger problems never need less
    big = _rows(n_rows=300, max_pos=999)
    assert ws(B.QSA_OP_TOPK, R(c), R(big), 0, 512) >= ws(B.QSA_OP_TOPK, R(c), R(q), 0, 512)


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, -1), ("page_size", 48, -1), ("page_size", 2, -1), ("n_kv_heads", 0, -1),
    ("head_dim", 96, -2), ("idx_dim", 24, -2), ("max_seq_len", 5000, -1),
    ("block_table", None, -1), ("seq_len", None, -1),
    ("block_size", 3, -1), ("block_size", 32, -1), ("block_size", -4, -1),
])
def test_cache_validation(libqsa, field, value, status):
    c = _cache(**{field: value})
    q = _rows()
    assert libqsa.qsa_pool_blocks(R(c), 8, 4, None) == status
    assert libqsa.qsa_index_scores(R(c), R(q), 8, 8, 4, 8, 512, None) == status


def test_call_validation(libqsa):
    c, q = _cache(), _rows()
    L = libqsa
    # pooling
    assert L.qsa_pool_blocks(R(c), None, 4, None) == -1
    assert L.qsa_pool_blocks(R(c), 8, -1, None) == -1
    assert L.qsa_pool_blocks(R(c), None, 0, None) == 0          # no-op, nothing enqueued
    # scores
    assert L.qsa_index_scores(R(c), R(q), 8, 8, 0, 8, 512, None) == -1     # heads
    assert L.qsa_index_scores(R(c), R(q), 8, 8, 9, 8, 512, None) == -1
    assert L.qsa_index_scores(R(c), R(q), 8, 8, 4, 8, 100, None) == -1     # ld < max_pos/4
    assert L.qsa_index_scores(R(c), R(_rows(max_pos=1000)), 8, 8, 4, 8, 512, None) == -1
    assert L.qsa_index_scores(R(c), R(_rows(seq_id=None)), 8, 8, 4, 8, 512, None) == -1
    # top-k
    ws = L.qsa_workspace_size(B.QSA_OP_TOPK, R(c), R(q), 0, 512)
    tk = L.qsa_topk_blocks
    assert tk(R(c), R(q), 8, 512, None, None, 0, 0, 8, 8, 8, ws, None) == -1      # top_k 0
    assert tk(R(c), R(q), 8, 512, None, None, 0, 2049, 8, 8, 8, ws, None) == -1   # > 2048
    assert tk(R(c), R(q), None, 0, None, 8, 4, 512, 8, 8, 8, ws, None) == -1      # fused, no q_idx
    assert tk(R(c), R(q), 8, 512, None, None, 0, 512, None, 8, 8, ws, None) == -1  # no sel
    assert tk(R(c), R(q), 8, 512, None, None, 0, 512, 8, 8, 8, ws - 1, None) == -3
    assert tk(R(c), R(q), 8, 512, None, None, 0, 512, 8, 8, None, ws, None) == -3
    # top-k that pools each row's newest block first: fused scoring only,
    # and the cache must hold the indexer keys
    tp = L.qsa_topk_blocks_pool_newest
    assert tp(R(_cache(kidx=None)), R(q), 8, 8, 4, 512, 8, 8, 8, ws, None) == -1
    assert tp(R(c), R(q), None, 8, 4, 512, 8, 8, 8, ws, None) == -1             # no q_idx
    assert tp(R(c), R(q), 8, 8, 4, 0, 8, 8, 8, ws, None) == -1                  # top_k 0
    assert tp(R(c), R(q), 8, 8, 4, 512, 8, 8, 8, ws - 1, None) == -3
    # attention
    wd = L.qsa_workspace_size(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 512)
    ad = L.qsa_attn_decode
    f = ctypes.c_float
    assert ad(R(c), R(q), 8, 15, 8, 8, 512, f(0.1), 8, 8, wd, None) == -1       # Hq % Hkv
    assert ad(R(c), R(q), 8, 16, 8, 8, 512, f(0.0), 8, 8, wd, None) == -1       # scale
    assert ad(R(c), R(q), 8, 16, 8, 8, 512, f(float("nan")), 8, 8, wd, None) == -1
    assert ad(R(c), R(q), 8, 16, None, 8, 512, f(0.1), 8, 8, wd, None) == -1
    assert ad(R(c), R(q), 8, 16, 8, 8, 512, f(0.1), 8, 8, wd - 1, None) == -3
    assert ad(R(c), R(q), 8, 64, 8, 8, 512, f(0.1), 8, 8, wd, None) == -2       # Hq*D > 4096
    assert L.qsa_dense_attn_decode(R(c), R(q), 8, 16, f(0.1), 8, None, 0, None) == -3
    wsh = L.qsa_workspace_size(B.QSA_OP_ATTN_DECODE_SHARED, R(c), R(q), 16, 512)
    sh = L.qsa_attn_decode_shared
    assert sh(R(c), R(q), 8, 16, 8, 8, None, 512, f(0.1), 8, 8, wsh, None) == -1   # no sel_of
    assert sh(R(c), R(q), 8, 16, 8, 8, 8, 512, f(0.1), 8, 8, wsh - 1, None) == -3
    assert sh(R(c), R(q), 8, 16, 8, 8, 8, 0, f(0.1), 8, 8, wsh, None) == -1       # top_k 0
    # indexer projections
    pj = L.qsa_index_project
    assert pj(R(c), R(q), 8, 100, 8, 8, 8, 4, 8, 8, 8, None) == -1        # h_dim % 64
    assert pj(R(c), R(q), 8, 0, 8, 8, 8, 4, 8, 8, 8, None) == -1
    assert pj(R(c), R(q), 8, 2048, 8, 8, 8, 0, 8, 8, 8, None) == -1       # no heads
    assert pj(R(c), R(q), 8, 2048, 8, 8, 8, 9, 8, 8, 8, None) == -1       # > 8 heads
    assert pj(R(c), R(q), None, 2048, 8, 8, 8, 4, 8, 8, 8, None) == -1    # no x
    assert pj(R(c), R(q), 8, 2048, 8, 8, 8, 4, 8, None, 8, None) == -1    # no kidx_out
    assert pj(R(_cache(dtype=0)), R(q), 8, 2048, 8, 8, 8, 4, 8, 8, 8, None) == -2  # f32
    # zero rows: valid and a no-op
    z = _rows(n_rows=0, seq_id=None, pos=None)
    assert L.qsa_attn_prefill(R(c), R(z), None, 16, 8, 8, 512, f(0.1), None, None, 0, None) == 0


@pytest.mark.parametrize("block", [0, 1, 2, 4, 8, 16])
def test_block_sizes_accepted(libqsa, block):
    """Block sizes 1..16 (0 = QSA's 4) are valid; a block longer than a page
    is not.  Finer blocks mean more candidates: the top-k workspace never
    shrinks as the block gets finer."""
    c, q = _cache(block_size=block), _rows()
    ws = libqsa.qsa_workspace_size
    assert ws(B.QSA_OP_TOPK, R(c), R(q), 0, 512) > 0
    assert ws(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 2048) > 0
    assert libqsa.qsa_pool_blocks(R(c), None, 0, None) == 0
    if block:
        coarser = _cache(block_size=min(16, 2 * block))
        assert ws(B.QSA_OP_TOPK, R(c), R(q), 0, 512) >= ws(B.QSA_OP_TOPK, R(coarser), R(q), 0, 512)
    small_page = _cache(block_size=16, page_size=8)
    assert libqsa.qsa_pool_blocks(R(small_page), 8, 4, None) == -1


def test_top_k_limit(libqsa):
    c, q = _cache(block_size=1), _rows()
    f = ctypes.c_float
    tk = libqsa.qsa_topk_blocks
    wsz = libqsa.qsa_workspace_size(B.QSA_OP_TOPK, R(c), R(q), 0, 2048)
    assert B.QSA_MAX_TOPK == 2048
    assert tk(R(c), R(q), None, 0, 8, 8, 4, 2049, 8, 8, 8, wsz, None) == -1
    assert tk(R(c), R(q), None, 0, 8, 8, 4, 0, 8, 8, 8, wsz, None) == -1
    at = libqsa.qsa_attn_decode
    wsa = libqsa.qsa_workspace_size(B.QSA_OP_ATTN_DECODE, R(c), R(q), 16, 2048)
    assert at(R(c), R(q), 8, 16, 8, 8, 2049, f(0.1), 8, 8, wsa, None) == -1


def test_release_build_has_no_debug_checks(libqsa):
    """qsa_debug_take reports QSA_ERR_UNSUPPORTED (and zero flags) on the
    release build, and rejects a null flags pointer."""
    f = ctypes.c_uint32(7)
    want = -2 if "debug" not in os.path.basename(B.LIB_PATH) else 0
    assert libqsa.qsa_debug_take(ctypes.byref(f)) == want
    assert f.value == 0
    assert libqsa.qsa_debug_take(None) == -1


def test_noalloc_decode_validates_before_launch(libqsa):
    """The no-allocation decode rejects invalid arguments on the host, like
    qsa_attn_decode (no GPU work happens on these paths)."""
    c, q = _cache(), _rows()
    f = libqsa.qsa_attn_decode_noalloc
    F = ctypes.c_float
    assert f(None, R(q), 8, 16, 8, 8, 512, F(0.1), 8, None) == -1          # no cache
    assert f(R(c), R(q), None, 16, 8, 8, 512, F(0.1), 8, None) == -1      # no q
    assert f(R(c), R(q), 8, 16, None, 8, 512, F(0.1), 8, None) == -1      # no sel
    assert f(R(c), R(q), 8, 16, 8, 8, 0, F(0.1), 8, None) == -1           # top_k < 1
    assert f(R(c), R(q), 8, 15, 8, 8, 512, F(0.1), 8, None) == -1         # Hq % Hkv
    assert f(R(c), R(q), 8, 16, 8, 8, 512, F(0.0), 8, None) == -1         # scale <= 0
