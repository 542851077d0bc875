"""Seeded synthetic workloads for the QSA hot path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no pooling, scoring, selection or attention).  Both the
GPU tests and the CPU oracle consume what it produces.

Input recipe (the pages print no data; the shapes follow the long-context
workloads they discuss, see the design notes):

* Q, K, V ~ N(0, 1), stored in the workload dtype (float32 or bfloat16).
* Indexer keys kidx and indexer queries q_idx lie on a grid: round(8 x) / 8
  clipped to [-4, 4], with x ~ N(0, 1) for keys and x ~ N(0, 1) + s_seq for
  queries, where s_seq in {-1, +1}^Di is one seeded direction per sequence.
  On this grid every float32 sum and product of the indexer is exact, so any
  summation order gives the same scores bit for bit.  The shared direction
  makes the planted needles win for every query; it also makes the rows of a
  sequence prefer some of the same blocks (about 30 % of two rows'
  selections coincide at 1M context).  Workloads with direction_scale 0
  draw x ~ N(0, 1) alone: their selections are independent across rows (the
  needles are then not guaranteed to be selected).
* Head weights w = (round(15 u) + 1) / 16 with u ~ U(0, 1): multiples of
  1/16 in [1/16, 1], never zero.
* Needle blocks: all 4 indexer keys of a 4-token span equal 3 * s_seq, which
  makes the block score far above every other block for every query that can
  see it (the generator does not check this; the tests do).  Needles are
  placed in 4-token units whatever the block size, so that workloads that
  differ only in the block size draw identical inputs.
* The KV cache is paged: page_size tokens per page; a sequence's pages are
  listed in block_table (a seeded permutation of the page pool when
  permute_pages is set, the identity otherwise).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

BLOCK_TOKENS = 4  # span length used to place needles (QSA's micro-block)


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str               # "decode", "prefill", "mtp" (multi-token decode) or
                            # "project" (the indexer projections alone)
    dtype: str              # "f32" or "bf16"
    n_seqs: int
    n_ctx: int              # tokens already cached before this step's rows
    n_new: int              # query rows per sequence (appended tokens)
    hq: int
    hkv: int
    d: int
    hi: int
    di: int
    top_k: int
    page_size: int = 64
    n_needles: int = 0      # per sequence, at seeded random depths
    needle_depths: tuple = ()  # fractions of the candidate range (decode)
    permute_pages: bool = False
    chunk: int = 0          # prefill chunk length; 0 = all rows in one step
    hidden: int = 0         # hidden size of the indexer projections ("project")
    seed: int = 0
    block: int = 4          # tokens per pooled block (1: token-granular selection)
    direction_scale: float = 1.0  # weight of the sequence direction in q_idx

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def total_len(self) -> int:
        return self.n_ctx + self.n_new

    @property
    def pages_per_seq(self) -> int:
        return -(-self.total_len // self.page_size)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads the method is measured on (mtp4_1m: four draft tokens of a
# multi-token decode step at 1M context sharing one selection).
WORKLOADS = {
    "tiny_decode": Workload(
        name="tiny_decode", mode="decode", dtype="f32", n_seqs=1, n_ctx=64,
        n_new=1, hq=4, hkv=1, d=32, hi=2, di=16, top_k=4, n_needles=1,
        seed=1001),
    "decode_8x32k": Workload(
        name="decode_8x32k", mode="decode", dtype="bf16", n_seqs=8,
        n_ctx=32768, n_new=1, hq=16, hkv=2, d=128, hi=4, di=64, top_k=512,
        n_needles=8, permute_pages=True, seed=1002),
    "decode_1m": Workload(
        name="decode_1m", mode="decode", dtype="bf16", n_seqs=1,
        n_ctx=1048576, n_new=1, hq=16, hkv=2, d=128, hi=4, di=64, top_k=512,
        needle_depths=(0.0, 0.25, 0.5, 0.75, 0.99), seed=1003),
    "mtp4_1m": Workload(
        name="mtp4_1m", mode="mtp", dtype="bf16", n_seqs=1,
        n_ctx=1048576, n_new=4, hq=16, hkv=2, d=128, hi=4, di=64, top_k=512,
        needle_depths=(0.0, 0.25, 0.5, 0.75, 0.99), seed=1006),
    "project_32k": Workload(
        name="project_32k", mode="project", dtype="bf16", n_seqs=1, n_ctx=0,
        n_new=32768, hq=16, hkv=2, d=128, hi=4, di=64, top_k=512, hidden=2048,
        seed=1007),
    "prefill_8k_at_128k": Workload(
        name="prefill_8k_at_128k", mode="prefill", dtype="bf16", n_seqs=1,
        n_ctx=131072, n_new=8192, hq=16, hkv=2, d=128, hi=4, di=64,
        top_k=512, n_needles=16, seed=1004),
    "prefill_1m": Workload(
        name="prefill_1m", mode="prefill", dtype="bf16", n_seqs=1, n_ctx=0,
        n_new=1048576, hq=16, hkv=2, d=128, hi=4, di=64, top_k=512,
        n_needles=32, chunk=32768, seed=1005),
    # the same prefill with indexer queries that share no direction: rows
    # select independently of each other (no reuse of selected blocks
    # across the rows of a chunk)
    "prefill_1m_indep": Workload(
        name="prefill_1m_indep", mode="prefill", dtype="bf16", n_seqs=1, n_ctx=0,
        n_new=1048576, hq=16, hkv=2, d=128, hi=4, di=64, top_k=512,
        n_needles=32, chunk=32768, seed=1005, direction_scale=0.0),
    # token-granular selection (block size 1) with the same 2,048-token
    # budget, on the same inputs as the block workloads they are named after
    "prefill_8k_at_128k_tok": Workload(
        name="prefill_8k_at_128k_tok", mode="prefill", dtype="bf16", n_seqs=1,
        n_ctx=131072, n_new=8192, hq=16, hkv=2, d=128, hi=4, di=64,
        top_k=2048, n_needles=16, seed=1004, block=1),
    "decode_1m_tok": Workload(
        name="decode_1m_tok", mode="decode", dtype="bf16", n_seqs=1,
        n_ctx=1048576, n_new=1, hq=16, hkv=2, d=128, hi=4, di=64, top_k=2048,
        needle_depths=(0.0, 0.25, 0.5, 0.75, 0.99), seed=1003, block=1),
    "decode_8x32k_tok": Workload(
        name="decode_8x32k_tok", mode="decode", dtype="bf16", n_seqs=8,
        n_ctx=32768, n_new=1, hq=16, hkv=2, d=128, hi=4, di=64, top_k=2048,
        n_needles=8, permute_pages=True, seed=1002, block=1),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def grid8(x: torch.Tensor) -> torch.Tensor:
    """round(8 x) / 8 clipped to [-4, 4] (exact in float32 and bfloat16)."""
    return torch.clamp(torch.round(x * 8.0) / 8.0, -4.0, 4.0)


@dataclass
class Cache:
    """Paged cache tensors of one workload (all on one device)."""
    wl: Workload
    k: torch.Tensor            # [n_pages, page, Hkv, D]
    v: torch.Tensor            # [n_pages, page, Hkv, D]
    kidx: torch.Tensor         # [n_pages, page, Di]
    kbar: torch.Tensor         # [n_pages, page/block, Di] (filled by pooling)
    block_table: torch.Tensor  # [n_seqs, pages_per_seq] int32
    seq_len: torch.Tensor      # [n_seqs] int32
    direction: torch.Tensor    # [n_seqs, Di] float32, entries +-1
    needles: list              # per sequence: list of needle block ids

    @property
    def n_pages(self) -> int:
        return self.k.shape[0]


def make_cache(wl: Workload, device="cpu", seed: int | None = None) -> Cache:
    """Draw the cache of workload wl (all n_ctx + n_new tokens present).

    Draw order from one generator: page permutation, K, V, kidx, the
    per-sequence directions, needle depths.
    """
    seed = wl.seed if seed is None else seed
    g = _gen(device, seed)
    dt = wl.torch_dtype
    pps = wl.pages_per_seq
    n_pages = wl.n_seqs * pps
    if wl.permute_pages:
        perm = torch.randperm(n_pages, generator=g, device=device)
    else:
        perm = torch.arange(n_pages, device=device)
    block_table = perm.view(wl.n_seqs, pps).to(torch.int32).contiguous()
    shape_kv = (n_pages, wl.page_size, wl.hkv, wl.d)
    k = torch.randn(shape_kv, generator=g, device=device).to(dt)
    v = torch.randn(shape_kv, generator=g, device=device).to(dt)
    kidx = grid8(torch.randn((n_pages, wl.page_size, wl.di), generator=g,
                             device=device)).to(dt)
    kbar = torch.zeros((n_pages, wl.page_size // wl.block, wl.di),
                       dtype=dt, device=device)
    direction = (torch.randint(0, 2, (wl.n_seqs, wl.di), generator=g,
                               device=device) * 2 - 1).to(torch.float32)
    seq_len = torch.full((wl.n_seqs,), wl.total_len, dtype=torch.int32,
                         device=device)

    # needles live among the blocks every query of the step can see
    # (decode) or among the blocks of the existing context (prefill with
    # existing context) or of the whole sequence (full prefill)
    if wl.mode == "decode":
        n_blocks_visible = (wl.total_len - 1) // BLOCK_TOKENS
    elif wl.mode == "mtp":  # the candidates of the draft rows' shared selection
        n_blocks_visible = wl.n_ctx // BLOCK_TOKENS
    elif wl.n_ctx > 0:
        n_blocks_visible = wl.n_ctx // BLOCK_TOKENS
    else:
        n_blocks_visible = wl.total_len // BLOCK_TOKENS
    needles = []
    for s in range(wl.n_seqs):
        if wl.needle_depths:
            ids = [min(int(dep * n_blocks_visible), n_blocks_visible - 1)
                   for dep in wl.needle_depths]
        else:
            ids = torch.randperm(n_blocks_visible, generator=g,
                                 device=device)[: wl.n_needles].tolist()
        ids = sorted(set(int(i) for i in ids))
        needles.append(ids)
        val = (3.0 * direction[s]).to(dt)
        for b in ids:
            for i in range(BLOCK_TOKENS):
                tok = BLOCK_TOKENS * b + i
                page = int(block_table[s, tok // wl.page_size])
                kidx[page, tok % wl.page_size] = val
    return Cache(wl=wl, k=k, v=v, kidx=kidx, kbar=kbar,
                 block_table=block_table, seq_len=seq_len,
                 direction=direction, needles=needles)


@dataclass
class Queries:
    """Query rows of one step."""
    seq_id: torch.Tensor   # [T] int32
    pos: torch.Tensor      # [T] int32 absolute positions
    q: torch.Tensor        # [T, Hq, D]
    q_idx: torch.Tensor    # [T, Hi, Di]
    w: torch.Tensor        # [T, Hi] float32

    @property
    def n(self) -> int:
        return int(self.pos.shape[0])


def make_queries(wl: Workload, cache: Cache, seq_id, pos, device="cpu",
                 seed: int | None = None) -> Queries:
    """Draw query rows at the given (seq_id, pos) pairs.

    Draw order: Q, the indexer query noise, the head-weight uniforms.
    """
    seed = (wl.seed + 7919) if seed is None else seed
    g = _gen(device, seed)
    seq_id = torch.as_tensor(seq_id, dtype=torch.int32, device=device)
    pos = torch.as_tensor(pos, dtype=torch.int32, device=device)
    n = int(pos.shape[0])
    dt = wl.torch_dtype
    q = torch.randn((n, wl.hq, wl.d), generator=g, device=device).to(dt)
    noise = torch.randn((n, wl.hi, wl.di), generator=g, device=device)
    direc = cache.direction.to(device)[seq_id.long()]            # [n, Di]
    q_idx = grid8(noise + wl.direction_scale * direc[:, None, :]).to(dt)
    u = torch.rand((n, wl.hi), generator=g, device=device)
    w = (torch.round(u * 15.0) + 1.0) / 16.0
    return Queries(seq_id=seq_id.contiguous(), pos=pos.contiguous(),
                   q=q.contiguous(), q_idx=q_idx.contiguous(),
                   w=w.to(torch.float32).contiguous())


def decode_rows(wl: Workload):
    """(seq_id, pos) of a decode step: the last token of every sequence."""
    seq_id = list(range(wl.n_seqs))
    pos = [wl.total_len - 1] * wl.n_seqs
    return seq_id, pos


def prefill_rows(wl: Workload, chunk_index: int = 0):
    """(seq_id, pos) of one prefill step (chunk) of sequence 0."""
    step = wl.chunk if wl.chunk else wl.n_new
    start = wl.n_ctx + chunk_index * step
    stop = min(start + step, wl.total_len)
    pos = list(range(start, stop))
    return [0] * len(pos), pos


def mtp_rows(wl: Workload):
    """(seq_id, pos, sel_of) of a multi-token decode step: the n_new draft
    tokens of every sequence (positions n_ctx .. n_ctx + n_new - 1).  The
    first draft row of each sequence comes first (rows 0 .. n_seqs - 1): the
    selection is made for it, and every draft row of the sequence reuses it
    (sel_of = the sequence's first row)."""
    seq_id = list(range(wl.n_seqs))
    pos = [wl.n_ctx] * wl.n_seqs
    sel_of = list(range(wl.n_seqs))
    for s in range(wl.n_seqs):
        for j in range(1, wl.n_new):
            seq_id.append(s)
            pos.append(wl.n_ctx + j)
            sel_of.append(s)
    return seq_id, pos, sel_of


@dataclass
class Projection:
    """Hidden states and indexer projection weights (one row per output)."""
    x: torch.Tensor    # [T, H]
    wq: torch.Tensor   # [Hi * Di, H]
    wk: torch.Tensor   # [Di, H]
    ww: torch.Tensor   # [Hi, H]


def make_projection(wl: Workload, rows: int, hidden: int, device="cpu", grid: bool = False,
                    seed: int | None = None) -> Projection:
    """Draw hidden states and projection weights.  grid=False: x ~ N(0, 1),
    weights ~ N(0, 1) / sqrt(H).  grid=True: x = round(8 N(0,1)) / 8 clipped
    to [-4, 4] and weights multiples of 1/16 in [-1, 1]; then every product
    is a multiple of 2^-7 of magnitude at most 4, and every sum of up to
    2^14 of them is exact in float32.  Draw order: x, wq, wk, ww."""
    g = _gen(device, (wl.seed + 104729) if seed is None else seed)
    dt = wl.torch_dtype

    def w_(n):
        r = torch.randn((n, hidden), generator=g, device=device)
        if grid:
            return torch.clamp(torch.round(r * 8.0) / 16.0, -1.0, 1.0).to(dt)
        return (r / hidden ** 0.5).to(dt)

    x = torch.randn((rows, hidden), generator=g, device=device)
    x = grid8(x) if grid else x
    return Projection(x=x.to(dt).contiguous(), wq=w_(wl.hi * wl.di).contiguous(),
                      wk=w_(wl.di).contiguous(), ww=w_(wl.hi).contiguous())


def step_rows(wl: Workload, chunk_index: int = 0):
    if wl.mode == "mtp":
        return mtp_rows(wl)[:2]
    if wl.mode == "project":
        return prefill_rows(wl, chunk_index)
    return decode_rows(wl) if wl.mode == "decode" else prefill_rows(wl, chunk_index)


def seq_view(cache: Cache, s: int, length: int | None = None):
    """Contiguous per-sequence copies (K, V, kidx) of the first length tokens.

    Gathers the sequence's pages through block_table; used only to hand the
    same inputs to the CPU oracle.
    """
    wl = cache.wl
    length = wl.total_len if length is None else length
    n_p = -(-length // wl.page_size)
    pages = cache.block_table[s, :n_p].long()
    k = cache.k[pages].reshape(-1, wl.hkv, wl.d)[:length]
    v = cache.v[pages].reshape(-1, wl.hkv, wl.d)[:length]
    kidx = cache.kidx[pages].reshape(-1, wl.di)[:length]
    return k, v, kidx
