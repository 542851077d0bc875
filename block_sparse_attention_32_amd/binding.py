"""ctypes binding of libqsa's C ABI (include/qsa.h).

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity, turned into raw pointers and passed with torch's current HIP
stream.  Every computation runs in the HIP library; if the library is not
built this module raises instead of computing anything elsewhere.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# QSA_LIB selects another build of the same library (the sanitized host
# build the ABI tests run against); the in-tree libqsa.so otherwise
LIB_PATH = os.environ.get("QSA_LIB") or os.path.join(_PKG, "libqsa.so")

QSA_BLOCK = 4
QSA_MAX_BLOCK = 16
QSA_BUDGET_TOKENS = 2048
QSA_MAX_TOPK = 2048
QSA_F32, QSA_BF16 = 0, 1
QSA_OP_TOPK, QSA_OP_ATTN_DECODE, QSA_OP_ATTN_PREFILL = 0, 1, 2
QSA_OP_DENSE_DECODE, QSA_OP_DENSE_PREFILL, QSA_OP_ATTN_DECODE_SHARED = 3, 4, 5
QSA_MAX_SHARED_LAG = 60

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace", -4: "hip error"}

SYMBOLS = (
    "qsa_pool_blocks", "qsa_index_project", "qsa_index_scores", "qsa_topk_blocks",
    "qsa_topk_blocks_pool_newest", "qsa_attn_decode",
    "qsa_attn_decode_shared", "qsa_attn_prefill", "qsa_dense_attn_decode",
    "qsa_dense_attn_prefill",
    "qsa_workspace_size", "qsa_status_string", "qsa_version", "qsa_debug_take",
    "qsa_attn_decode_noalloc",
)
QSA_NOALLOC_SCRATCH_BYTES = 16 << 20
QSA_DEBUG_BAD_PAGE, QSA_DEBUG_BAD_ROW, QSA_DEBUG_BAD_SEL = 1, 2, 4
DEBUG_LIB_PATH = os.path.join(_PKG, "libqsa_debug.so")


class QsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("n_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kidx", ctypes.c_void_p), ("kbar", ctypes.c_void_p),
    ]


class _Queries(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int32), ("max_pos", ctypes.c_int32),
        ("seq_id", ctypes.c_void_p), ("pos", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqsa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                "python -m block_sparse_attention_32_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_size_t, ctypes.c_float)
        sig = {
            "qsa_pool_blocks": [P, P, I32, P],
            "qsa_index_scores": [P, P, P, P, I32, P, I64, P],
            "qsa_index_project": [P, P, P, I32, P, P, P, I32, P, P, P, P],
            "qsa_topk_blocks": [P, P, P, I64, P, P, I32, I32, P, P, P, SZ, P],
            "qsa_topk_blocks_pool_newest": [P, P, P, P, I32, I32, P, P, P, SZ, P],
            "qsa_attn_decode": [P, P, P, I32, P, P, I32, F, P, P, SZ, P],
            "qsa_attn_decode_shared": [P, P, P, I32, P, P, P, I32, F, P, P, SZ, P],
            "qsa_attn_prefill": [P, P, P, I32, P, P, I32, F, P, P, SZ, P],
            "qsa_dense_attn_decode": [P, P, P, I32, F, P, P, SZ, P],
            "qsa_dense_attn_prefill": [P, P, P, I32, F, P, P, SZ, P],
            "qsa_workspace_size": [I32, P, P, I32, I32],
            "qsa_debug_take": [P],
            "qsa_attn_decode_noalloc": [P, P, P, I32, P, P, I32, F, P, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_size_t if name == "qsa_workspace_size" else ctypes.c_int
        L.qsa_status_string.argtypes = [ctypes.c_int]
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


_DT = {torch.float32: QSA_F32, torch.bfloat16: QSA_BF16}


class CacheView:
    """qsa_cache over torch tensors (keeps them alive while in use).

    k, v: [n_pages, page, Hkv, D]; kidx: [n_pages, page, Di];
    kbar: [n_pages, page/B, Di] (B tokens per pooled block: its shape gives
    B); block_table: [n_seqs, max_pages] int32; seq_len: [n_seqs] int32;
    max_seq_len: host upper bound of seq_len.
    """

    def __init__(self, k, v, kidx, kbar, block_table, seq_len, max_seq_len: int):
        for t, n in ((k, "k"), (v, "v"), (kidx, "kidx"), (kbar, "kbar")):
            _check(t, n, dtype=k.dtype, device=k.device)
        _check(block_table, "block_table", torch.int32, k.device)
        _check(seq_len, "seq_len", torch.int32, k.device)
        if k.dtype not in _DT:
            raise ValueError("cache dtype must be float32 or bfloat16")
        n_pages, page, hkv, d = k.shape
        if kbar.dim() != 3 or kbar.shape[1] < 1 or page % kbar.shape[1] != 0:
            raise ValueError("kbar must be [n_pages, page_size / block, Di]")
        self.block = page // kbar.shape[1]
        self.tensors = (k, v, kidx, kbar, block_table, seq_len)
        self.device = k.device
        self.dtype = k.dtype
        self.head_dim = d
        self.n_kv_heads = hkv
        self.s = _Cache(
            dtype=_DT[k.dtype], page_size=page, block_size=self.block,
            n_kv_heads=hkv, head_dim=d,
            idx_dim=kidx.shape[-1], n_seqs=block_table.shape[0],
            max_pages_per_seq=block_table.shape[1], max_seq_len=int(max_seq_len),
            n_pages=n_pages, block_table=_ptr(block_table), seq_len=_ptr(seq_len),
            k=_ptr(k), v=_ptr(v), kidx=_ptr(kidx), kbar=_ptr(kbar))

    @classmethod
    def from_cache(cls, c) -> "CacheView":
        """From a workloads.Cache (all of its tokens present)."""
        return cls(c.k, c.v, c.kidx, c.kbar, c.block_table, c.seq_len, c.wl.total_len)

    @property
    def ref(self):
        return ctypes.byref(self.s)


class QueriesView:
    """qsa_queries over int32 device tensors seq_id, pos; max_pos is a host
    upper bound of pos."""

    def __init__(self, seq_id, pos, max_pos: int):
        _check(seq_id, "seq_id", torch.int32)
        _check(pos, "pos", torch.int32, seq_id.device)
        self.tensors = (seq_id, pos)
        self.n_rows = int(pos.shape[0])
        self.s = _Queries(n_rows=self.n_rows, max_pos=int(max_pos),
                          seq_id=_ptr(seq_id), pos=_ptr(pos))

    @property
    def ref(self):
        return ctypes.byref(self.s)


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise QsaError(name, st)


def qsa_debug_take() -> int:
    """Device-data check bits recorded by a debug build since the last call
    (synchronises); raises QsaError on the release build."""
    f = ctypes.c_uint32(0)
    _call("qsa_debug_take", ctypes.byref(f))
    return int(f.value)


def qsa_workspace_size(op: int, cache: CacheView, queries: QueriesView,
                       n_q_heads: int = 0, top_k: int = 0) -> int:
    return int(lib().qsa_workspace_size(op, cache.ref, queries.ref, n_q_heads, top_k))


def workspace(op: int, cache: CacheView, queries: QueriesView, n_q_heads: int = 0,
              top_k: int = 0) -> torch.Tensor:
    """A zero-filled workspace of the size `op` needs (at least 256 bytes)."""
    n = max(256, qsa_workspace_size(op, cache, queries, n_q_heads, top_k))
    return torch.zeros(n, dtype=torch.uint8, device=cache.device)


def qsa_pool_blocks(cache: CacheView, blk_begin: torch.Tensor, max_new_blocks: int,
                    stream=None):
    _check(blk_begin, "blk_begin", torch.int32, cache.device)
    _call("qsa_pool_blocks", cache.ref, _ptr(blk_begin), int(max_new_blocks), _stream(stream))


def qsa_index_scores(cache: CacheView, queries: QueriesView, q_idx, w, scores, ld=None,
                     stream=None):
    _check(q_idx, "q_idx", cache.dtype, cache.device)
    _check(w, "w", torch.float32, cache.device)
    _check(scores, "scores", torch.float32, cache.device)
    ld = scores.shape[-1] if ld is None else ld
    _call("qsa_index_scores", cache.ref, queries.ref, _ptr(q_idx), _ptr(w),
          int(q_idx.shape[1]), _ptr(scores), int(ld), _stream(stream))


def qsa_topk_blocks(cache: CacheView, queries: QueriesView, top_k: int, sel, n_sel, ws,
                    scores=None, ld=None, q_idx=None, w=None, stream=None):
    _check(sel, "sel", torch.int32, cache.device)
    _check(n_sel, "n_sel", torch.int32, cache.device)
    _check(ws, "ws", None, cache.device)
    hi = 0
    if scores is not None:
        _check(scores, "scores", torch.float32, cache.device)
        ld = scores.shape[-1] if ld is None else ld
    else:
        _check(q_idx, "q_idx", cache.dtype, cache.device)
        _check(w, "w", torch.float32, cache.device)
        hi = int(q_idx.shape[1])
        ld = 0
    _call("qsa_topk_blocks", cache.ref, queries.ref, _ptr(scores), int(ld), _ptr(q_idx),
          _ptr(w), hi, int(top_k), _ptr(sel), _ptr(n_sel), _ptr(ws),
          ws.numel() * ws.element_size(), _stream(stream))


def qsa_topk_blocks_pool_newest(cache: CacheView, queries: QueriesView, top_k: int, sel,
                                n_sel, ws, q_idx, w, stream=None):
    _check(sel, "sel", torch.int32, cache.device)
    _check(n_sel, "n_sel", torch.int32, cache.device)
    _check(ws, "ws", None, cache.device)
    _check(q_idx, "q_idx", cache.dtype, cache.device)
    _check(w, "w", torch.float32, cache.device)
    _call("qsa_topk_blocks_pool_newest", cache.ref, queries.ref, _ptr(q_idx), _ptr(w),
          int(q_idx.shape[1]), int(top_k), _ptr(sel), _ptr(n_sel), _ptr(ws),
          ws.numel() * ws.element_size(), _stream(stream))


def _attn(name, cache, queries, q, sel, n_sel, top_k, scale, out, ws, stream):
    _check(q, "q", cache.dtype, cache.device)
    _check(out, "out", cache.dtype, cache.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if sel is None:
        _call(name, cache.ref, queries.ref, _ptr(q), int(q.shape[1]), ctypes.c_float(scale),
              _ptr(out), _ptr(ws), wsb, _stream(stream))
    else:
        _check(sel, "sel", torch.int32, cache.device)
        _check(n_sel, "n_sel", torch.int32, cache.device)
        _call(name, cache.ref, queries.ref, _ptr(q), int(q.shape[1]), _ptr(sel), _ptr(n_sel),
              int(top_k), ctypes.c_float(scale), _ptr(out), _ptr(ws), wsb, _stream(stream))


def qsa_index_project(cache, queries, x, wq, wk, ww, q_idx, w, kidx_out=None, stream=None):
    """Indexer projections of the rows' hidden states x [T, H]: q_idx [T, Hi,
    Di], w [T, Hi] float32, and each row's indexer key written into kidx_out
    (default: the cache's kidx).  Weights [out, H], bfloat16."""
    for t, n in ((x, "x"), (wq, "wq"), (wk, "wk"), (ww, "ww"), (q_idx, "q_idx")):
        _check(t, n, cache.dtype, cache.device)
    _check(w, "w", torch.float32, cache.device)
    kidx_out = cache.tensors[2] if kidx_out is None else kidx_out
    _check(kidx_out, "kidx_out", cache.dtype, cache.device)
    _call("qsa_index_project", cache.ref, queries.ref, _ptr(x), int(x.shape[1]), _ptr(wq),
          _ptr(wk), _ptr(ww), int(ww.shape[0]), _ptr(q_idx), _ptr(kidx_out), _ptr(w),
          _stream(stream))


def qsa_attn_decode(cache, queries, q, sel, n_sel, top_k, scale, out, ws, stream=None):
    _attn("qsa_attn_decode", cache, queries, q, sel, n_sel, top_k, scale, out, ws, stream)


def qsa_attn_decode_noalloc(cache, queries, q, sel, n_sel, top_k, scale, out, stream=None):
    """qsa_attn_decode on the library's static scratch (no workspace)."""
    _check(q, "q", cache.dtype, cache.device)
    _check(out, "out", cache.dtype, cache.device)
    _check(sel, "sel", torch.int32, cache.device)
    _check(n_sel, "n_sel", torch.int32, cache.device)
    _call("qsa_attn_decode_noalloc", cache.ref, queries.ref, _ptr(q), int(q.shape[1]), _ptr(sel),
          _ptr(n_sel), int(top_k), ctypes.c_float(scale), _ptr(out), _stream(stream))


def qsa_attn_decode_shared(cache, queries, q, sel, n_sel, sel_of, top_k, scale, out, ws,
                           stream=None):
    """Decode rows reusing the selection of row sel_of[i] (draft tokens of a
    multi-token step): see qsa_attn_decode_shared in include/qsa.h."""
    _check(q, "q", cache.dtype, cache.device)
    _check(out, "out", cache.dtype, cache.device)
    for t, n in ((sel, "sel"), (n_sel, "n_sel"), (sel_of, "sel_of")):
        _check(t, n, torch.int32, cache.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _call("qsa_attn_decode_shared", cache.ref, queries.ref, _ptr(q), int(q.shape[1]), _ptr(sel),
          _ptr(n_sel), _ptr(sel_of), int(top_k), ctypes.c_float(scale), _ptr(out), _ptr(ws),
          wsb, _stream(stream))


def qsa_attn_prefill(cache, queries, q, sel, n_sel, top_k, scale, out, ws=None, stream=None):
    _attn("qsa_attn_prefill", cache, queries, q, sel, n_sel, top_k, scale, out, ws, stream)


def qsa_dense_attn_decode(cache, queries, q, scale, out, ws, stream=None):
    _attn("qsa_dense_attn_decode", cache, queries, q, None, None, 0, scale, out, ws, stream)


def qsa_dense_attn_prefill(cache, queries, q, scale, out, ws=None, stream=None):
    _attn("qsa_dense_attn_prefill", cache, queries, q, None, None, 0, scale, out, ws, stream)
