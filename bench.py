"""Benchmark of the QSA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic query rows,
with the cache already resident in HBM:
  decode : pool the newest complete block, fused indexer scores and exact
           top-k (one call) -> split-K sparse attention (one query row per
           sequence)
  prefill: for every chunk of the prefill in order: pool the chunk's complete
           blocks -> fused scores + top-k -> per-row sparse attention
The default workload is the full 1M-token prefill (32 chunks of 32,768 rows).

Prints one JSON line: query-tokens/s, per-call kernel times from HIP events
on the launch stream, the roofline of the dominant kernel, the dense-GQA
comparison on the same inputs, and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_attention_32_amd import binding as B  # noqa: E402
from block_sparse_attention_32_amd import workloads as W  # noqa: E402
from block_sparse_attention_32_amd.rocprof_summary import source_hash, traffic_for  # noqa: E402

METRIC = "QSA decode/prefill query-tokens/s at 128K & 1M ctx; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events around each API call of the timed steps (torch's current
    stream, which is the stream every libqsa call is launched on)."""

    def __init__(self):
        self.pairs = {}

    def wrap(self, name, fn, *a, **kw):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn(*a, **kw)
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def avg_us(self):
        return {k: 1e3 * float(np.mean([s.elapsed_time(e) for s, e in v]))
                for k, v in self.pairs.items()}


# ------------------------------------------------------------------ decode

def run_decode(wl: W.Workload, steps: int, warmup: int, dev, dense: bool = True):
    """One step = pool the newest complete block, fused indexer scores and
    exact top-k (one call: the block is pooled by the top-k workgroup that
    scores it) -> split-K sparse attention, for one query row per sequence."""
    from block_sparse_attention_32_amd import pipeline as P
    log(f"[bench] drawing {wl.name} cache on {dev}")
    cache = W.make_cache(wl, device=dev)
    seq_id, pos = W.decode_rows(wl)
    qs = W.make_queries(wl, cache, seq_id, pos, device=dev)
    cv = B.CacheView.from_cache(cache)
    rows = B.QueriesView(qs.seq_id, qs.pos, max(pos))
    bk = wl.block
    n_blocks = wl.total_len // bk
    P.pool_all(cv, wl.n_seqs, n_blocks, dev)               # set-up, untimed
    step = P.QsaStep(cv, rows, qs.q, qs.q_idx, qs.w, wl.top_k, wl.scale, "decode")

    def one(timer=None):
        call = timer.wrap if timer else (lambda name, fn, *a, **k: fn(*a, **k))
        call("topk", step.select_pooling_newest)   # pools, scores and selects
        call("attn", step.attend)

    wall, kern = _timed(one, steps, warmup)
    n_sel = step.n_sel.cpu().numpy()
    n_tok = int(sum(bk * int(n) + p % bk + 1 for n, p in zip(n_sel, pos)))
    cand = sum(p // bk for p in pos)
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        # the pooled keys streamed, plus each row's newest block pooled
        "topk": {"bytes": (cand + len(pos) * (bk + 1)) * wl.di * esz, "bound": "hbm",
                 "kernel": "topk_kernel",
                 "files": ("index.hip", "index.hpp", "select.hpp", "common.hpp")},
        "attn": {"bytes": n_tok * wl.hkv * wl.d * esz * 2, "bound": "hbm",
                 "kernel": "attn_mfma_kernel",
                 "files": ("attention_mfma.hip", "attention.hpp", "common.hpp")},
    }
    dense_ms = None
    if dense:
        ds = P.DenseStep(cv, rows, qs.q, wl.scale, "decode")
        dense_ms = _dense_time(ds.run, max(5, steps // 4))
    ctx = {"rows": rows.n_rows, "cache": cache, "qs": qs, "pos": pos, "launches": 1,
           "dense_ms": dense_ms, "dense_note": "split-K flash-decode over all tokens",
           "step": step}
    return wall, kern, work, ctx


def run_mtp(wl: W.Workload, steps: int, warmup: int, dev, dense: bool = True):
    """One multi-token decode step: pool the newest complete block -> fused
    scores and exact top-k for each sequence's first draft row -> split-K
    sparse attention of every draft row over that selection plus its own
    recent tokens."""
    from block_sparse_attention_32_amd import pipeline as P
    log(f"[bench] drawing {wl.name} cache on {dev}")
    cache = W.make_cache(wl, device=dev)
    seq_id, pos, sel_of = W.mtp_rows(wl)
    qs = W.make_queries(wl, cache, seq_id, pos, device=dev)
    cv = B.CacheView.from_cache(cache)
    rows = B.QueriesView(qs.seq_id, qs.pos, max(pos))
    bk = wl.block
    n_blocks = wl.total_len // bk
    P.pool_all(cv, wl.n_seqs, n_blocks, dev)               # set-up, untimed
    sel_of_t = torch.tensor(sel_of, dtype=torch.int32, device=dev)
    step = P.MtpStep(cv, rows, qs.q, qs.q_idx, qs.w, sel_of_t, wl.n_seqs, wl.top_k, wl.scale)
    newest = torch.full((wl.n_seqs,), n_blocks - 1, dtype=torch.int32, device=dev)

    def one(timer=None):
        call = timer.wrap if timer else (lambda name, fn, *a, **k: fn(*a, **k))
        call("pool", B.qsa_pool_blocks, cv, newest, 1)
        call("topk", step.select)
        call("attn", step.attend)

    wall, kern = _timed(one, steps, warmup)
    n_sel = step.n_sel.cpu().numpy()
    n_tok = int(sum(bk * int(n_sel[s]) + p - bk * (pos[s] // bk) + 1
                    for s, p in zip(sel_of, pos)))
    cand = sum(pos[s] // bk for s in range(wl.n_seqs))
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        "topk": {"bytes": cand * wl.di * esz, "bound": "hbm", "kernel": "topk_kernel",
                 "files": ("index.hip", "index.hpp", "select.hpp", "common.hpp")},
        "attn": {"bytes": n_tok * wl.hkv * wl.d * esz * 2, "bound": "hbm",
                 "kernel": "attn_mfma_kernel",
                 "files": ("attention_mfma.hip", "attention.hpp", "common.hpp")},
        "pool": {"bytes": wl.n_seqs * (bk + 1) * wl.di * esz, "bound": "hbm",
                 "kernel": "pool_kernel", "files": ("index.hip", "index.hpp", "common.hpp")},
    }
    dense_ms = None
    if dense:
        ds = P.DenseStep(cv, rows, qs.q, wl.scale, "decode")
        dense_ms = _dense_time(ds.run, max(5, steps // 4))
    ctx = {"rows": rows.n_rows, "cache": cache, "qs": qs, "pos": pos, "sel_of": sel_of,
           "launches": 1, "dense_ms": dense_ms, "step": step,
           "dense_note": "split-K flash-decode of every draft row over all its tokens"}
    return wall, kern, work, ctx


def run_project(wl: W.Workload, steps: int, warmup: int, dev):
    """One step = the indexer projections of one prefill chunk of rows:
    q_idx, w and the rows' indexer keys (into the paged cache) from hidden
    states of size wl.hidden."""
    log(f"[bench] drawing {wl.name} on {dev}")
    cache = W.make_cache(wl, device=dev)
    seq_id, pos = W.prefill_rows(wl, 0)
    pj = W.make_projection(wl, len(pos), wl.hidden, device=dev)
    cv = B.CacheView.from_cache(cache)
    rows = B.QueriesView(torch.tensor(seq_id, dtype=torch.int32, device=dev),
                         torch.tensor(pos, dtype=torch.int32, device=dev), max(pos))
    q_idx = torch.empty((len(pos), wl.hi, wl.di), dtype=wl.torch_dtype, device=dev)
    w = torch.empty((len(pos), wl.hi), dtype=torch.float32, device=dev)

    def one(timer=None):
        call = timer.wrap if timer else (lambda name, fn, *a, **k: fn(*a, **k))
        call("project", B.qsa_index_project, cv, rows, pj.x, pj.wq, pj.wk, pj.ww, q_idx, w)

    wall, kern = _timed(one, steps, warmup)
    t, h = len(pos), wl.hidden
    n = wl.hi * wl.di + wl.di + wl.hi
    esz = 2
    work = {"project": {"bytes": t * h * esz + n * h * esz + t * (wl.hi * wl.di + wl.di) * esz
                                 + t * wl.hi * 4,
                        "flops": 2 * t * h * n, "bound": "hbm", "kernel": "project_kernel",
                        "files": ("project.hip", "project.hpp", "common.hpp")}}
    ctx = {"rows": t, "cache": cache, "pos": pos, "proj": pj, "launches": 1, "dense_ms": None}
    return wall, kern, work, ctx


STEP_MS: list = []  # per-step times (HIP events, per group of steps) after the timed region


def _timed(one, steps, warmup):
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the spread of the step times, in a separate run: HIP events around
    # groups of m steps (an event between microsecond steps slows them down
    # by a few microseconds, so short steps are timed 20 at a time)
    m = 20 if wall / steps < 1e-3 else 1
    n = 10 if m > 1 else max(1, min(steps, 10))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        for _ in range(m):
            one()
        ev[i + 1].record()
    torch.cuda.synchronize()
    global STEP_MS
    STEP_MS = [ev[i].elapsed_time(ev[i + 1]) / m for i in range(n)]
    timer = Timer()
    for _ in range(max(1, min(steps, 50))):
        one(timer)
    torch.cuda.synchronize()
    return wall, timer


def _dense_time(fn, reps):
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return 1e3 * (time.perf_counter() - t0) / reps


# ------------------------------------------------------------------ prefill

def run_prefill(wl: W.Workload, steps: int, warmup: int, dev, dense: bool = True,
                dense_budget_s: float = 60.0, overlap: bool = False):
    """One step = the whole prefill of wl: every chunk of query rows in
    order (pool the chunk's new blocks -> fused scores + top-k -> per-row
    sparse attention; with overlap the attention of chunk c runs on a second
    stream beside the selection of chunk c+1).  The existing context (if any)
    is pooled at set-up."""
    from block_sparse_attention_32_amd import pipeline as P
    log(f"[bench] drawing {wl.name} cache on {dev}")
    cache = W.make_cache(wl, device=dev)
    cv = B.CacheView.from_cache(cache)
    bk = wl.block
    n_chunks = max(1, -(-wl.n_new // (wl.chunk or wl.n_new)))
    chunks = []
    for ci in range(n_chunks):
        seq_id, pos = W.prefill_rows(wl, ci)
        qs = W.make_queries(wl, cache, seq_id, pos, device=dev, seed=wl.seed + 7919 + ci)
        rows = B.QueriesView(qs.seq_id, qs.pos, max(pos))
        st = P.QsaStep(cv, rows, qs.q, qs.q_idx, qs.w, wl.top_k, wl.scale, "prefill")
        b0 = pos[0] // bk
        begin = torch.full((1,), b0, dtype=torch.int32, device=dev)
        chunks.append((st, begin, (pos[-1] + 1) // bk - b0, pos, qs, rows))
    if wl.n_ctx:
        P.pool_all(cv, 1, wl.n_ctx // bk, dev)              # set-up, untimed

    sched = P.ChunkedPrefill(cv, [(c[0], c[1], c[2]) for c in chunks], overlap=overlap)

    def one(timer=None):
        sched.run(timer.wrap if timer else None)

    wall, kern = _timed(one, steps, warmup)
    rows_total = sum(len(c[3]) for c in chunks)
    n_tok = 0
    cand = 0
    dense_flop = []
    for st, _, _, pos, _, _ in chunks:
        ns = st.n_sel.cpu().numpy().astype(np.int64)
        p_ = np.asarray(pos, dtype=np.int64)
        n_tok += int((bk * ns + p_ % bk + 1).sum())
        cand += int((p_ // bk).sum())
        dense_flop.append(4.0 * wl.hq * wl.d * float((p_ + 1).sum()))
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        "attn": {"bytes": n_tok * wl.hkv * wl.d * esz * 2, "flops": 4 * wl.hq * wl.d * n_tok,
                 "bound": "hbm", "kernel": "attn_mfma_kernel",
                 "files": ("attention_mfma.hip", "attention.hpp", "common.hpp")},
        "topk": {"flops": 2 * wl.hi * wl.di * cand, "bound": "mfma",
                 "kernel": "pidx_kernel+pidx_tau_kernel+pidx_select_wave_kernel+pidx_select_kernel",
                 "files": ("index_mfma.hip", "index.hpp", "select.hpp", "common.hpp")},
        "pool": {"bytes": (wl.n_new // bk) * (bk + 1) * wl.di * esz, "bound": "hbm",
                 "kernel": "pool_kernel", "files": ("index.hip", "index.hpp", "common.hpp")},
    }
    # dense GQA attention over the same rows, chunk by chunk in order while
    # the next chunk's projected time fits the budget; the rest is
    # extrapolated by flops
    ctx = {"rows": rows_total, "cache": cache, "chunks": chunks, "launches": n_chunks,
           "dense_ms": None}
    if not dense:
        return wall, kern, work, ctx
    measured = {}
    t_start = time.perf_counter()
    for ci in range(n_chunks):
        if measured:
            per_flop = sum(measured.values()) / sum(dense_flop[c] for c in measured)
            left = dense_budget_s - (time.perf_counter() - t_start)
            if per_flop * dense_flop[ci] * 1e-3 > left:
                break
        ds = P.DenseStep(cv, chunks[ci][5], chunks[ci][4].q, wl.scale, "prefill")
        measured[ci] = _dense_time(ds.run, 1)
        del ds
    per_flop = sum(measured.values()) / sum(dense_flop[c] for c in measured)
    dense_ms = per_flop * sum(dense_flop)
    note = ("dense causal GQA over all chunks" if len(measured) == n_chunks else
            f"dense causal GQA on chunks {sorted(measured)} of {n_chunks}, "
            "extrapolated by flops")
    ctx.update(dense_ms=dense_ms, dense_note=note,
               dense_tflops=sum(dense_flop) / (dense_ms * 1e-3) / 1e12)
    return wall, kern, work, ctx


# ------------------------------------------------------------------ memory

def memory_report(wl, ctx, dev):
    """Device memory of the mask-free hand-off against a materialised kq_mask
    for the largest call of the step (the last prefill chunk, or the decode
    rows): the selection and the workspaces the library needs (sel, n_sel,
    top-k and attention workspaces) versus a float16 [rows x keys] mask of
    the same rows, which is allocated and filled here so that its footprint
    is measured (free device memory before and after), not just computed."""
    if wl.mode == "prefill":
        st, pos = ctx["chunks"][-1][0], ctx["chunks"][-1][3]
    else:
        st, pos = ctx["step"], ctx["pos"]
    rows, keys = len(pos), max(pos) + 1
    free_bytes = sum(t.numel() * t.element_size()
                     for t in (st.sel, st.n_sel, st.ws_topk, st.ws_attn))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0 = torch.cuda.mem_get_info(dev)[0]
    mask = torch.empty((rows, keys), dtype=torch.float16, device=dev)
    mask.fill_(float("-inf"))
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info(dev)[0]
    del mask
    torch.cuda.empty_cache()
    need = rows * keys * 2
    seen = int(free0 - free1)
    return {"rows": rows, "keys": keys, "kq_mask_bytes": need,
            # below the allocator's granularity the free-memory reading does not move
            "kq_mask_measured_bytes": seen if seen >= need // 2 else None,
            "mask_free_bytes": int(free_bytes),
            "how": "float16 [rows x keys] mask allocated and filled (measured as the drop in "
                   "free device memory); mask-free = sel + n_sel + top-k and attention "
                   "workspaces of the same call"}


# ------------------------------------------------------------------ CPU oracle

def measured_peaks(dev, reps=10):
    """What this GPU achieves beside the published peaks: a plain 1 GiB
    device-to-device copy (bytes read + written per second) and an
    8192^3 bf16 GEMM (torch.matmul, i.e. the vendor BLAS).  Context for the
    roofline fractions, which stay against the published peaks."""
    def timed(fn):
        for _ in range(3):
            fn()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e-3 / reps

    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    copy_gbs = 2 * src.numel() / t_copy / 1e9
    del src, dst
    n = 8192
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g).contiguous()
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(a, b, out=c))
    gemm_tflops = 2 * n ** 3 / t_mm / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": round(copy_gbs, 1), "bf16_gemm_tflops": round(gemm_tflops, 1),
            "how": "1 GiB device copy (read + write bytes) and an 8192^3 bf16 torch.matmul, "
                   f"{reps} timed repetitions each (library kernels: lower bounds on what "
                   "the chip sustains)"}


def cpu_baseline(wl, ctx, budget_s=12.0):
    """The oracle (numpy float64, one thread) on a bounded sample of the same
    workload, scaled to query-tokens/s of the whole job."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    cache = ctx["cache"]
    log("[bench] cpu oracle: copying the cache to host")
    seqs = {}

    def seq(s):
        if s not in seqs:
            k, v, kidx = W.seq_view(cache, s)
            seqs[s] = [k.float().cpu().numpy(), v.float().cpu().numpy(),
                       kidx.double().cpu().numpy(), None]
        return seqs[s]

    if wl.mode == "mtp":
        return cpu_baseline_mtp(wl, ctx, seq, budget_s)
    if wl.mode == "project":
        return cpu_baseline_project(wl, ctx, budget_s)
    if wl.mode == "decode":
        qs, pos = ctx["qs"], ctx["pos"]
        rows = [(s, t, qs.q[i], qs.q_idx[i], qs.w[i]) for i, (s, t) in
                enumerate(zip(qs.seq_id.cpu().tolist(), pos))][:64]
        for s, *_ in rows:
            e = seq(s)
            if e[3] is None:
                e[3] = O.pool_blocks(e[2], wl.dtype, block=wl.block)   # set-up, untimed
        pool_s = 0.0
        sample = f"decode rows of {wl.name}, repeated"
    else:
        # whole-job pooling once (timed), then a seeded uniform sample of rows
        e = seq(0)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            e[3] = O.pool_blocks(e[2], wl.dtype, block=wl.block)
            pool_s = time.perf_counter() - t0
        rng = np.random.default_rng(wl.seed + 1)
        rows = []
        for _ in range(4096):
            ci = int(rng.integers(len(ctx["chunks"])))
            _, _, _, pos, qs, _ = ctx["chunks"][ci]
            i = int(rng.integers(len(pos)))
            rows.append((0, pos[i], qs.q[i], qs.q_idx[i], qs.w[i]))
        sample = f"seeded uniform sample of {wl.name} rows"
    rows = [(s, t, q.double().cpu().numpy(), qi.double().cpu().numpy(), w.double().cpu().numpy())
            for s, t, q, qi, w in rows]
    done, el = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while el < budget_s:
            for s, t, q, qi, w in rows:
                k, v, _, kbar = seq(s)
                if wl.mode == "decode":
                    bk = wl.block
                    nb = (t + 1) // bk
                    kbar[nb - 1:nb] = O.pool_blocks(seq(s)[2][: bk * nb], wl.dtype, nb - 1, nb,
                                                    block=bk)
                O.qsa_row(k, v, kbar, q, qi, w, t, wl.top_k, wl.scale, wl.block)
                done += 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
    per_row = el / done
    job_s = pool_s + per_row * ctx["rows"]
    return {"value": round(ctx["rows"] / job_s, 3), "unit": "query-tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} {sample} (score, select, attend; {el:.1f} s)"
                      + (f" + whole-job pooling {pool_s:.1f} s; whole job "
                         f"extrapolated as pooling + rows x mean row time"
                         if wl.mode != "decode" else "") +
                      "; numpy float64 single-threaded"}


def cpu_baseline_project(wl, ctx, budget_s):
    """Oracle of the projections (numpy float64 matrix products, one thread)
    on batches of the same rows, scaled to rows/s."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    pj = ctx["proj"]
    x = pj.x.double().cpu().numpy()
    wq, wk, ww = (t.double().cpu().numpy() for t in (pj.wq, pj.wk, pj.ww))
    batch = 256
    done, el = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while el < budget_s:
            i = done % (x.shape[0] - batch)
            O.index_project(x[i:i + batch], wq, wk, ww, wl.hi, wl.dtype)
            done += batch
            el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows of {wl.name} in batches of {batch} ({el:.1f} s); numpy "
                      "float64 single-threaded"}


def cpu_baseline_mtp(wl, ctx, seq, budget_s):
    """Oracle of a multi-token decode step: one selection per sequence, then
    every draft row attends it plus its own recent tokens; repeated steps."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    qs, pos, sel_of = ctx["qs"], ctx["pos"], ctx["sel_of"]
    seq_ids = qs.seq_id.cpu().tolist()
    q = qs.q.double().cpu().numpy()
    qi = qs.q_idx.double().cpu().numpy()
    w = qs.w.double().cpu().numpy()
    for s in set(seq_ids):
        e = seq(s)
        if e[3] is None:
            e[3] = O.pool_blocks(e[2], wl.dtype, block=wl.block)   # set-up, untimed
    done, el = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while el < budget_s:
            sels = {}
            for i, s in enumerate(seq_ids):
                k, v, _, kbar = seq(s)
                r = sel_of[i]
                if r not in sels:
                    sels[r] = O.qsa_select_row(kbar, qi[r], w[r], pos[r], wl.top_k, wl.block)
                O.attend(q[i], k, v, O.token_set_shared(sels[r], pos[r], pos[i], wl.block),
                         wl.scale)
                done += 1
            el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} draft rows of {wl.name} ({done // len(seq_ids)} repeated steps: "
                      f"select once per sequence, attend every row; {el:.1f} s); numpy float64 "
                      "single-threaded"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="prefill_1m", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-GQA comparison")
    ap.add_argument("--overlap", action="store_true",
                    help="prefill: run each chunk's attention on a second stream, beside the "
                         "next chunk's selection (per-kernel times then overlap)")
    ap.add_argument("--no-memory", action="store_true",
                    help="skip the mask-free vs materialised-kq_mask memory measurement")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable copy bandwidth and bf16 GEMM rate "
                         "(also skipped with --copy-calibration)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the QSA path "
              "here is single-GPU by design.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    decode = wl.mode in ("decode", "mtp")
    short = decode or wl.mode == "project"  # microsecond steps: many of them
    steps = args.steps if args.steps is not None else (200 if short else 3)
    warmup = args.warmup if args.warmup is not None else (20 if short else 1)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if wl.mode == "project":
        wall, timer, work, ctx = run_project(wl, steps, warmup, dev)
    elif wl.mode == "mtp":
        wall, timer, work, ctx = run_mtp(wl, steps, warmup, dev, dense=not args.no_dense)
    elif decode:
        wall, timer, work, ctx = run_decode(wl, steps, warmup, dev, dense=not args.no_dense)
    else:
        wall, timer, work, ctx = run_prefill(wl, steps, warmup, dev, dense=not args.no_dense,
                                             overlap=args.overlap)
    kern_call = timer.avg_us()                      # per API call
    calls_per_step = ctx["launches"]
    kern = {k: v * calls_per_step for k, v in kern_call.items()}   # per step
    ms = 1e3 * wall / steps
    value = ctx["rows"] / (wall / steps)
    dom = max((k for k in kern if k in work), key=kern.get)
    wk = work[dom]
    src_hash = source_hash(*wk["files"])
    avg_us = kern_call[dom]
    if wk["bound"] == "hbm":
        per_launch = wk["bytes"] / calls_per_step
        achieved, peak, unit = per_launch / (avg_us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        per_launch = wk["flops"] / calls_per_step
        achieved, peak, unit = per_launch / (avg_us * 1e-6) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    roof = {"bound": wk["bound"], "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic_for(wk["kernel"].split("+")[0], wl.name, src_hash),
            "kernel": wk["kernel"], "algorithmic_per_launch": per_launch,
            "avg_launch_us": round(avg_us, 2), "source_hash": src_hash}
    cfg = {"workload": wl.name, "n_seqs": wl.n_seqs, "context": wl.n_ctx,
           "new_tokens": wl.n_new, "query_rows_per_step": ctx["rows"],
           "chunk": (wl.chunk or wl.n_new) if not decode else None,
           "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "idx_heads": wl.hi, "idx_dim": wl.di,
           "top_k": wl.top_k, "block_tokens": wl.block, "page_size": wl.page_size,
           "parallelism": "single-gpu"}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "step_ms": {"min": round(min(STEP_MS), 4), "median": round(float(np.median(STEP_MS)), 4),
                    "max": round(max(STEP_MS), 4)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic", "config": cfg,
        "roofline": roof,
        "kernels_us_per_step": {k: round(v, 2) for k, v in kern.items()},
    }
    if wl.mode == "project":
        pw = work["project"]
        t_us = kern["project"]
        out["projection_mfma"] = {"flops_per_step": pw["flops"],
                                  "achieved_tflops": round(pw["flops"] / (t_us * 1e-6) / 1e12, 1),
                                  "peak_tflops": BF16_PEAK_TFLOPS,
                                  "frac": round(pw["flops"] / (t_us * 1e-6) / 1e12
                                                / BF16_PEAK_TFLOPS, 4)}
    elif not decode:
        tk = work["topk"]
        t_us = kern["topk"]
        out["indexer_mfma"] = {"kernels": tk["kernel"], "flops_per_step": tk["flops"],
                               "achieved_tflops": round(tk["flops"] / (t_us * 1e-6) / 1e12, 1),
                               "peak_tflops": BF16_PEAK_TFLOPS,
                               "frac": round(tk["flops"] / (t_us * 1e-6) / 1e12
                                             / BF16_PEAK_TFLOPS, 4)}
    if ctx["dense_ms"] is not None:
        out["dense_gqa"] = {"ms_per_step": round(ctx["dense_ms"], 4),
                            "speedup_sparse_over_dense": round(ctx["dense_ms"] / ms, 2),
                            "how": ctx.get("dense_note", "")}
        if "dense_tflops" in ctx:
            out["dense_gqa"]["achieved_tflops"] = round(ctx["dense_tflops"], 1)
    # a counter run's only device copy must be the calibration copy
    if not args.no_peaks and not args.copy_calibration:
        mp = measured_peaks(dev)
        out["measured_peaks"] = mp
        meas = mp["hbm_copy_gbs"] if unit == "GB/s" else mp["bf16_gemm_tflops"]
        roof["measured_peak"] = meas
        roof["frac_of_measured_peak"] = round(achieved / meas, 4)
        for key in ("indexer_mfma", "projection_mfma"):
            if key in out:
                out[key]["frac_of_measured_peak"] = round(
                    out[key]["achieved_tflops"] / mp["bf16_gemm_tflops"], 4)
        if "achieved_tflops" in out.get("dense_gqa", {}):
            out["dense_gqa"]["frac_of_measured_peak"] = round(
                out["dense_gqa"]["achieved_tflops"] / mp["bf16_gemm_tflops"], 4)
    if not args.no_memory and wl.mode != "project":
        out["memory"] = memory_report(wl, ctx, dev)
    out["cpu_baseline"] = None if args.no_cpu else cpu_baseline(wl, ctx)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
