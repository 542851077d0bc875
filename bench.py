"""Benchmark of the QSA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic query rows,
with the cache already resident in HBM:
  decode : pool the newest complete block, fused indexer scores and exact
           top-k (one call) -> split-K sparse attention (one query row per
           sequence)
  prefill: for every chunk of the prefill in order: pool the chunk's complete
           blocks -> fused scores + top-k -> per-row sparse attention

With no --workload, every configuration of the method is measured in one
run -- tiny_decode, decode_8x32k, decode_1m, prefill_8k_at_128k, prefill_1m,
and prefill_1m_indep (the 1M prefill with independent selections) -- and
the headline (metric, value, roofline, cpu_baseline) is the full 1M-token
prefill; the others are records under "configs".  --workload NAME measures
one workload only.

Prints one JSON line: query-tokens/s, per-call kernel times from HIP events
on the launch stream, the roofline of the dominant call, the roofline of the
whole step, the dense-GQA comparison on the same inputs, and the CPU oracle
on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

if __name__ != "__mp_main__":
    # spawned CPU-oracle workers need numpy and the oracle only
    import torch

    from block_sparse_attention_32_amd import binding as B
    from block_sparse_attention_32_amd import workloads as W
    from block_sparse_attention_32_amd.rocprof_summary import source_hash, traffic_for

METRIC = "QSA decode/prefill query-tokens/s at 128K & 1M ctx; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X published fp32 vector
HEADLINE = "prefill_1m"
ALL_WORKLOADS = ("tiny_decode", "decode_8x32k", "decode_1m", "prefill_8k_at_128k", "prefill_1m",
                 "prefill_1m_indep")
MAX_CPU_WORKERS = 16           # host cores one GPU's share of a box may use


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

def run_decode(wl, steps: int, warmup: int, dev, dense: bool = True, graph: bool = False):
    """One step = pool the newest complete block, fused indexer scores and
    exact top-k (one call: the block is pooled by the top-k workgroup that
    scores it) -> split-K sparse attention, for one query row per sequence.
    With graph the step's two calls are captured once in a HIP graph and the
    timed steps replay it (the per-call event times stay eager calls)."""
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

    def eager(timer=None):
        call = timer.wrap if timer else (lambda name, fn, *a, **k: fn(*a, **k))
        call("topk", step.select_pooling_newest)   # pools, scores and selects
        call("attn", step.attend)

    one = eager
    if graph:
        eager()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            eager()
        torch.cuda.synchronize()

        def one(timer=None):
            if timer is not None:
                eager(timer)
            else:
                g.replay()

    wall, kern = _timed(one, steps, warmup)
    n_sel = step.n_sel.cpu().numpy()
    n_tok = int(sum(bk * int(n) + p % bk + 1 for n, p in zip(n_sel, pos)))
    cand = sum(p // bk for p in pos)
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        # the pooled keys streamed, plus each row's newest block pooled
        "topk": {"bytes": (cand + len(pos) * (bk + 1)) * wl.di * esz, "bound": "hbm",
                 "flops": 2 * wl.hi * wl.di * cand, "kernel": "topk_kernel",
                 "files": ("topk.hpp", "index_device.hpp", "index.hpp", "select.hpp",
                           "common.hpp")},
        # every attended token's K and V rows: no reuse inside a decode step
        "attn": {"bytes": n_tok * wl.hkv * wl.d * esz * 2, "bound": "hbm",
                 "flops": 4 * wl.hq * wl.d * n_tok, "kernel": "attn_mfma_kernel",
                 "files": ("attention_mfma.hip", "attention.hpp", "common.hpp")},
    }
    dense_ms = None
    if dense:
        ds = P.DenseStep(cv, rows, qs.q, wl.scale, "decode")
        dense_ms = _dense_time(ds.run, max(5, steps // 4))
    ctx = {"rows": rows.n_rows, "cache": cache, "qs": qs, "pos": pos, "launches": 1,
           "dense_ms": dense_ms, "dense_note": "split-K flash-decode over all tokens",
           "step": step, "graph": graph}
    return wall, kern, work, ctx


def run_mtp(wl, steps: int, warmup: int, dev, dense: bool = True):
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
                 "files": ("topk.hpp", "index_device.hpp", "index.hpp", "select.hpp",
                           "common.hpp")},
        # the draft rows share their selection: its blocks are read once
        "attn": {"bytes": (bk * int(n_sel[0]) + max(pos) - bk * (pos[0] // bk) + 1)
                 * wl.hkv * wl.d * esz * 2 * wl.n_seqs,
                 "flops": 4 * wl.hq * wl.d * n_tok, "bound": "hbm",
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


def run_project(wl, steps: int, warmup: int, dev):
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
                        "flops": 2 * t * h * n, "bound": "mfma", "kernel": "project_kernel",
                        "files": ("project.hip", "project.hpp", "common.hpp")}}
    ctx = {"rows": t, "cache": cache, "pos": pos, "proj": pj, "launches": 1, "dense_ms": None}
    return wall, kern, work, ctx


def _timed(one, steps, warmup):
    """(wall seconds of exactly `steps` steps, Timer of the per-call events,
    per-step times of a separate run).  The timed region holds no events."""
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
    step_ms = [ev[i].elapsed_time(ev[i + 1]) / m for i in range(n)]
    timer = Timer()
    for _ in range(max(1, min(steps, 50))):
        one(timer)
    torch.cuda.synchronize()
    timer.step_ms = step_ms
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

def run_prefill(wl, steps: int, warmup: int, dev, dense: bool = True,
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
    distinct_blocks = 0     # distinct (block) entries each attention launch reads
    dense_flop = []
    for st, _, _, pos, _, _ in chunks:
        ns = st.n_sel.cpu().numpy().astype(np.int64)
        p_ = np.asarray(pos, dtype=np.int64)
        n_tok += int((bk * ns + p_ % bk + 1).sum())
        cand += int((p_ // bk).sum())
        own = torch.as_tensor(p_ // bk, device=st.sel.device)
        ids = torch.cat([st.sel[st.sel >= 0].long(), own])
        distinct_blocks += int(torch.unique(ids).numel())
        dense_flop.append(4.0 * wl.hq * wl.d * float((p_ + 1).sum()))
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        # bytes: the K and V rows of the distinct blocks a launch reads (the
        # compulsory traffic: a block several rows select need be fetched
        # once); the per-row gather is in "gather_bytes"
        "attn": {"bytes": distinct_blocks * bk * wl.hkv * wl.d * esz * 2,
                 "gather_bytes": n_tok * wl.hkv * wl.d * esz * 2,
                 "flops": 4 * wl.hq * wl.d * n_tok, "kernel": "attn_mfma_kernel",
                 "files": ("attention_mfma.hip", "attention.hpp", "common.hpp")},
        # the pooled keys of a chunk are read once per launch
        "topk": {"flops": 2 * wl.hi * wl.di * cand,
                 "bytes": sum((c[3][-1] // bk) * wl.di * esz for c in chunks),
                 "kernel": "pidx_kernel+pidx_tau_wave_kernel+pidx_select_wave_kernel+pidx_select_kernel",
                 "files": ("index_mfma.hip", "index_device.hpp", "index.hpp", "select.hpp",
                           "common.hpp")},
        "pool": {"bytes": (wl.n_new // bk) * (bk + 1) * wl.di * esz,
                 "kernel": "pool_kernel", "files": ("index.hip", "index_device.hpp", "index.hpp",
                                                    "common.hpp")},
    }
    ctx = {"rows": rows_total, "cache": cache, "chunks": chunks, "launches": n_chunks,
           "dense_ms": None}
    if not dense:
        return wall, kern, work, ctx
    # dense GQA attention over the same rows, chunk by chunk in order while
    # the next chunk's projected time fits the budget; the rest is
    # extrapolated by flops
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


# ------------------------------------------------------------------ rooflines

def call_roofline(work_item, calls_per_step, avg_us, workload, fp32=False):
    """Roofline of one library call: its algorithmic bytes and flops per
    launch give the two lower bounds bytes / HBM peak and flops / MFMA peak;
    the larger is the bound, and frac = that time / the measured launch
    time (<= 1 by construction of a lower bound)."""
    per_b = work_item.get("bytes", 0) / calls_per_step
    per_f = work_item.get("flops", 0) / calls_per_step
    peak_f = FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS
    t_hbm = per_b / (HBM_PEAK_GBS * 1e9)
    t_mfma = per_f / (peak_f * 1e12)
    t = avg_us * 1e-6
    if t_hbm >= t_mfma:
        bound, achieved, peak, unit = "hbm", per_b / t / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", per_f / t / 1e12, peak_f, "TFLOP/s"
    frac = achieved / peak
    if frac > 1.0:
        raise RuntimeError(f"roofline fraction {frac:.3f} > 1 for {work_item['kernel']}: the "
                           "algorithmic work model is not a lower bound")
    src_hash = source_hash(*work_item["files"])
    r = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
         "frac": round(frac, 4),
         "traffic": traffic_for(work_item["kernel"].split("+")[0], workload, src_hash),
         "kernel": work_item["kernel"], "avg_launch_us": round(avg_us, 2),
         "algorithmic_bytes_per_launch": int(per_b), "algorithmic_flops_per_launch": int(per_f),
         "source_hash": src_hash}
    if "gather_bytes" in work_item:
        g = work_item["gather_bytes"] / calls_per_step
        r["gather_bytes_per_launch"] = int(g)
        r["gather_gbs"] = round(g / t / 1e9, 1)
    if r["traffic"]:
        r["traffic_gbs"] = round(r["traffic"] / t / 1e9, 1)
        r["traffic_frac_of_hbm_peak"] = round(r["traffic"] / t / 1e9 / HBM_PEAK_GBS, 4)
    return r


def step_roofline(work, ms, fp32=False):
    """The whole step against the roofline: the sum over its calls of each
    call's lower bound (max of bytes / HBM peak and flops / MFMA peak),
    divided by the measured step time (all launches, gaps included)."""
    peak_f = FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS
    t_roof = 0.0
    for w in work.values():
        t_roof += max(w.get("bytes", 0) / (HBM_PEAK_GBS * 1e9),
                      w.get("flops", 0) / (peak_f * 1e12))
    frac = t_roof / (ms * 1e-3)
    if frac > 1.0:
        raise RuntimeError(f"step roofline fraction {frac:.3f} > 1")
    return {"t_roof_ms": round(t_roof * 1e3, 5), "frac": round(frac, 4),
            "how": "sum over the step's calls of max(algorithmic bytes / 8 TB/s, flops / "
                   f"{peak_f:g} TFLOP/s), divided by the measured step time"}


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


# ------------------------------------------------------------------ CPU oracle

def cpu_workers() -> int:
    """Worker processes for the CPU oracle: one per host core this process
    may run on, at most one GPU's share of a box."""
    return max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))


def _attach(specs):
    """Views of the arrays the parent wrote to memory-mapped files
    {name: (path, shape, dtype)}; pooled keys are copy-on-write (a decode
    worker re-pools into its private copy)."""
    return {key: np.memmap(path, dtype=dt, mode="c" if key.startswith("kbar") else "r",
                           shape=tuple(shape))
            for key, (path, shape, dt) in specs.items()}


def _oracle_worker(job):
    """CPU-oracle worker (one process per core, BLAS on one thread): runs
    the oracle on its rows and returns ([(row tag, seconds)], wall-clock
    start, wall-clock end) of its work (process start-up excluded).  Decode
    rows first re-pool their sequence's newest block, as a decode step
    does."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    arrs = _attach(job["shm"])
    out = []
    with threadpool_limits(limits=1):
        w0 = time.time()
        out = _oracle_rows(O, arrs, job)
        return out, w0, time.time()


def _oracle_rows(O, arrs, job):
    out = []
    t_start = time.perf_counter()
    while True:
        for tag, s, t, q, qi, w in job["rows"]:
            t0 = time.perf_counter()
            k, v, kbar = arrs[f"k{s}"], arrs[f"v{s}"], arrs[f"kbar{s}"]
            if job["decode"]:
                bk = job["block"]
                nb = (t + 1) // bk
                kbar[nb - 1:nb] = O.pool_blocks(arrs[f"kidx{s}"][: bk * nb], job["dtype"],
                                                nb - 1, nb, block=bk)
            O.qsa_row(k, v, kbar, q, qi, w, t, job["top_k"], job["scale"], job["block"])
            out.append((tag, time.perf_counter() - t0))
            if time.perf_counter() - t_start >= job["budget_s"] and not job["full"]:
                return out
        if job["full"] or time.perf_counter() - t_start >= job["budget_s"]:
            return out


def _stratified_prefill_rows(wl, ctx):
    """Rows of the 1M prefill for the sampled CPU baseline: the first and
    last four rows of every chunk (every t mod 4 at both chunk edges), 14
    evenly spaced rows inside every chunk, rows t <= 2,051 (selection covers
    the whole context), and the first row after each needle (the first that
    can select it): about 750 rows, some 16 s of oracle work."""
    chunks = ctx["chunks"]
    picks = set()
    for ci, c in enumerate(chunks):
        pos = c[3]
        for i in list(range(4)) + list(range(len(pos) - 4, len(pos))):
            picks.add((ci, i))
        for j in range(1, 15):
            picks.add((ci, j * len(pos) // 15))
    first, clen = chunks[0][3][0], len(chunks[0][3])

    def add(t):  # the row at position t, if the prefill has one
        ci = (t - first) // clen
        if t >= first and ci < len(chunks) and t - chunks[ci][3][0] < len(chunks[ci][3]):
            picks.add((ci, t - chunks[ci][3][0]))

    for t in (0, 1, 2, 3, 1023, 2047, 2048, 2049, 2050, 2051):
        add(t)
    for b in ctx["cache"].needles[0]:
        add(4 * (b + 1))
    return sorted(picks)


def cpu_baseline(wl, ctx, budget_s=12.0):
    """The oracle (numpy float64) on the host cores, one worker process per
    core: decode steps repeated, the 8K-row prefill in full, the 1M prefill
    on a stratified sample (whole job extrapolated with a linear model of
    the row time in t, the row's position)."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import oracle as O
    cache = ctx["cache"]
    ncore = cpu_workers()
    log(f"[bench] cpu oracle: copying the cache to host ({ncore} workers)")
    if wl.mode == "decode":
        seqs = list(range(wl.n_seqs))
    else:
        seqs = [0]
    specs = {}
    tmp = tempfile.mkdtemp(prefix="qsa_oracle_")

    def share(key, arr):
        path = os.path.join(tmp, key + ".bin")
        mm = np.memmap(path, dtype=arr.dtype, mode="w+", shape=arr.shape)
        mm[...] = arr
        mm.flush()
        del mm
        specs[key] = (path, arr.shape, arr.dtype.str)

    try:
        pool_s = 0.0
        for s in seqs:
            k, v, kidx = W.seq_view(cache, s)
            kidx = kidx.double().cpu().numpy()
            share(f"k{s}", k.float().cpu().numpy())
            share(f"v{s}", v.float().cpu().numpy())
            share(f"kidx{s}", kidx)
            if wl.mode == "decode":
                kbar = O.pool_blocks(kidx, wl.dtype, block=wl.block)   # set-up, untimed
            else:
                t0 = time.perf_counter()     # the step pools every block (prefill): timed
                kbar = O.pool_blocks(kidx, wl.dtype, block=wl.block)
                pool_s += time.perf_counter() - t0
            share(f"kbar{s}", kbar)

        def row_of(qs, i, tag, s, t):
            return (tag, s, t, qs.q[i].double().cpu().numpy(), qs.q_idx[i].double().cpu().numpy(),
                    qs.w[i].double().cpu().numpy())

        base = {"shm": specs, "top_k": wl.top_k, "scale": wl.scale, "block": wl.block,
                "dtype": wl.dtype}
        if wl.mode == "decode":
            qs, pos = ctx["qs"], ctx["pos"]
            sid = qs.seq_id.cpu().tolist()
            rows = [row_of(qs, i, i, sid[i], pos[i]) for i in range(len(pos))]
            nw = min(ncore, len(rows))
            jobs = [dict(base, rows=rows[j::nw], decode=True, full=False, budget_s=budget_s)
                    for j in range(nw)]
        else:
            if len(ctx["chunks"]) == 1:        # one chunk: every row, in full
                c = ctx["chunks"][0]
                rows = [row_of(c[4], i, i, 0, c[3][i]) for i in range(len(c[3]))]
                full = True
            else:
                picks = _stratified_prefill_rows(wl, ctx)
                rows = [row_of(ctx["chunks"][ci][4], i, (ci, i), 0, ctx["chunks"][ci][3][i])
                        for ci, i in picks]
                full = True
            nw = min(ncore, len(rows))
            # longest rows first, each to the least-loaded worker (a row's
            # cost grows with its position t)
            load, parts = [0.0] * nw, [[] for _ in range(nw)]
            for r in sorted(rows, key=lambda r: -r[2]):
                j = int(np.argmin(load))
                parts[j].append(r)
                load[j] += 20000.0 + r[2]
            jobs = [dict(base, rows=parts[j], decode=False, full=full, budget_s=budget_s)
                    for j in range(nw)]
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                              "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"
        try:
            ctxmp = mp.get_context("spawn")
            with ctxmp.Pool(nw) as pool:
                got = pool.map(_oracle_worker, jobs)
            res = [g[0] for g in got]
            # the makespan of the workers' compute (process start-up excluded)
            wall = max(g[2] for g in got) - min(g[1] for g in got)
        finally:
            for k, val in env.items():
                if val is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = val
    finally:
        shutil.rmtree(tmp, ignore_errors=True)

    if wl.mode == "decode":
        # worker j repeats its rows; a step's time is the slowest worker's
        # per-step time
        per_step = max(sum(dt for _, dt in r) / max(1, len(r) // max(1, len(jobs[j]["rows"])))
                       for j, r in enumerate(res))
        n_steps = min(len(r) // max(1, len(jobs[j]["rows"])) for j, r in enumerate(res))
        return {"value": round(len(ctx["pos"]) / per_step, 3), "unit": "query-tokens/s",
                "cores": nw, "kind": "oracle",
                "sample": f"{n_steps}+ repeated decode steps of {wl.name} ({len(ctx['pos'])} "
                          f"row(s) per step over {nw} worker process(es), one BLAS thread "
                          "each; newest block re-pooled per step); numpy float64"}
    times = [dt for r in res for _, dt in r]
    if len(ctx["chunks"]) == 1:
        job_s = pool_s + wall
        return {"value": round(ctx["rows"] / job_s, 3), "unit": "query-tokens/s",
                "cores": nw, "kind": "oracle",
                "sample": f"every row of {wl.name} ({len(times)} rows over {nw} worker "
                          f"processes, one BLAS thread each, {wall:.1f} s) + pooling "
                          f"{pool_s:.2f} s; numpy float64"}
    # sampled: row time ~ a + b * t (scoring and sorting grow with the
    # candidate count); whole job = pooling + sum of predicted row times over
    # the workers at the parallel efficiency the sample reached
    tag_t = {(ci, i): ctx["chunks"][ci][3][i] for ci, i in _stratified_prefill_rows(wl, ctx)}
    ts = np.array([tag_t[tag] for r in res for tag, _ in r], dtype=np.float64)
    ys = np.array(times)
    a, b = np.linalg.lstsq(np.stack([np.ones_like(ts), ts], 1), ys, rcond=None)[0]
    all_t = np.concatenate([np.asarray(c[3], dtype=np.float64) for c in ctx["chunks"]])
    pred = float(np.sum(a + b * all_t))
    eff = min(1.0, (ys.sum() / nw) / wall)
    job_s = pool_s + pred / (nw * eff)
    return {"value": round(float(ctx["rows"] / job_s), 3), "unit": "query-tokens/s",
            "cores": nw, "kind": "oracle",
            "sample": f"stratified sample of {len(ys)} rows of {wl.name} (first and last 4 rows "
                      "and 14 evenly spaced rows of each of its chunks, rows t <= 2,051, the "
                      "first row after each needle) "
                      f"over {nw} worker processes, one BLAS thread each ({wall:.1f} s); whole "
                      f"job extrapolated: pooling {pool_s:.1f} s + row time fitted as "
                      f"{a * 1e3:.2f} ms + {b * 1e9:.1f} ns x t summed over every row, "
                      f"divided by {nw} workers at the sample's parallel efficiency {eff:.2f}; "
                      "numpy float64"}


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


def cpu_baseline_mtp(wl, ctx, budget_s):
    """Oracle of a multi-token decode step: one selection per sequence, then
    every draft row attends it plus its own recent tokens; repeated steps."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    cache = ctx["cache"]
    qs, pos, sel_of = ctx["qs"], ctx["pos"], ctx["sel_of"]
    seq_ids = qs.seq_id.cpu().tolist()
    q = qs.q.double().cpu().numpy()
    qi = qs.q_idx.double().cpu().numpy()
    w = qs.w.double().cpu().numpy()
    seqs = {}
    for s in set(seq_ids):
        k, v, kidx = W.seq_view(cache, s)
        seqs[s] = (k.float().cpu().numpy(), v.float().cpu().numpy(),
                   O.pool_blocks(kidx.double().cpu().numpy(), wl.dtype, block=wl.block))
    done, el = 0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while el < budget_s:
            sels = {}
            for i, s in enumerate(seq_ids):
                k, v, kbar = seqs[s]
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


# ------------------------------------------------------------------ one workload

def measure(wl, steps, warmup, args, dev, cpu=True, dense=True, memory=True):
    """The record of one workload: throughput, step-time spread, per-call
    times, rooflines, dense comparison, memory and the CPU oracle."""
    decode = wl.mode in ("decode", "mtp")
    if wl.mode == "project":
        wall, timer, work, ctx = run_project(wl, steps, warmup, dev)
    elif wl.mode == "mtp":
        wall, timer, work, ctx = run_mtp(wl, steps, warmup, dev, dense=dense)
    elif decode:
        wall, timer, work, ctx = run_decode(wl, steps, warmup, dev, dense=dense,
                                            graph=args.graph)
    else:
        wall, timer, work, ctx = run_prefill(wl, steps, warmup, dev, dense=dense,
                                             overlap=args.overlap)
    kern_call = timer.avg_us()                      # per API call
    calls_per_step = ctx["launches"]
    kern = {k: v * calls_per_step for k, v in kern_call.items()}   # per step
    ms = 1e3 * wall / steps
    value = ctx["rows"] / (wall / steps)
    fp32 = wl.dtype == "f32"
    rooflines = {k: call_roofline(work[k], calls_per_step, kern_call[k], wl.name, fp32)
                 for k in kern if k in work}
    dom = max(rooflines, key=lambda k: kern[k])
    cfg = {"workload": wl.name, "n_seqs": wl.n_seqs, "context": wl.n_ctx,
           "new_tokens": wl.n_new, "query_rows_per_step": ctx["rows"],
           "chunk": (wl.chunk or wl.n_new) if not decode else None,
           "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "idx_heads": wl.hi, "idx_dim": wl.di,
           "top_k": wl.top_k, "block_tokens": wl.block, "page_size": wl.page_size,
           "direction_scale": wl.direction_scale, "parallelism": "single-gpu",
           "hip_graph": bool(ctx.get("graph", False))}
    step_ms = timer.step_ms
    rec = {
        "value": round(value, 1), "unit": "query-tokens/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "step_ms": {"min": round(min(step_ms), 5), "median": round(float(np.median(step_ms)), 5),
                    "max": round(max(step_ms), 5)},
        "dtype": wl.dtype, "config": cfg,
        "roofline": rooflines[dom],
        "step_roofline": step_roofline({k: work[k] for k in kern if k in work}, ms, fp32),
        "calls_roofline": {k: {kk: r[kk] for kk in ("bound", "achieved", "unit", "frac",
                                                    "avg_launch_us")}
                           for k, r in rooflines.items()},
        "kernels_us_per_step": {k: round(v, 3) for k, v in kern.items()},
    }
    if wl.mode == "project":
        pw = work["project"]
        t_us = kern["project"]
        rec["projection_mfma"] = {"flops_per_step": pw["flops"],
                                  "achieved_tflops": round(pw["flops"] / (t_us * 1e-6) / 1e12, 1),
                                  "peak_tflops": BF16_PEAK_TFLOPS,
                                  "frac": round(pw["flops"] / (t_us * 1e-6) / 1e12
                                                / BF16_PEAK_TFLOPS, 4)}
    elif not decode:
        tk = work["topk"]
        t_us = kern["topk"]
        rec["indexer_mfma"] = {"kernels": tk["kernel"], "flops_per_step": tk["flops"],
                               "achieved_tflops": round(tk["flops"] / (t_us * 1e-6) / 1e12, 1),
                               "peak_tflops": BF16_PEAK_TFLOPS,
                               "frac": round(tk["flops"] / (t_us * 1e-6) / 1e12
                                             / BF16_PEAK_TFLOPS, 4)}
    if ctx["dense_ms"] is not None:
        rec["dense_gqa"] = {"ms_per_step": round(ctx["dense_ms"], 4),
                            "speedup_sparse_over_dense": round(ctx["dense_ms"] / ms, 2),
                            "how": ctx.get("dense_note", "")}
        if "dense_tflops" in ctx:
            rec["dense_gqa"]["achieved_tflops"] = round(ctx["dense_tflops"], 1)
            rec["dense_gqa"]["frac"] = round(ctx["dense_tflops"] / BF16_PEAK_TFLOPS, 4)
    if memory and wl.mode != "project":
        rec["memory"] = memory_report(wl, ctx, dev)
    if cpu:
        if wl.mode == "project":
            rec["cpu_baseline"] = cpu_baseline_project(wl, ctx, 10.0)
        elif wl.mode == "mtp":
            rec["cpu_baseline"] = cpu_baseline_mtp(wl, ctx, 10.0)
        else:
            rec["cpu_baseline"] = cpu_baseline(wl, ctx, 20.0 if wl.name == HEADLINE else 8.0)
    else:
        rec["cpu_baseline"] = None
    del ctx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def default_steps(wl, steps, warmup):
    short = wl.mode in ("decode", "mtp", "project")   # microsecond steps: many of them
    return (steps if steps is not None else (200 if short else 3),
            warmup if warmup is not None else (20 if short else 1))


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the headline workload (others: their defaults, at "
                         "least this many)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None, choices=sorted(W.WORKLOADS),
                    help="measure this workload only (default: every configuration, headline "
                         f"{HEADLINE})")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-GQA comparison")
    ap.add_argument("--graph", action="store_true",
                    help="decode: replay the step from a HIP graph (captured once)")
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
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = [args.workload] if args.workload else list(ALL_WORKLOADS)
    head_name = args.workload or HEADLINE
    records = {}
    for name in names:
        wl = W.WORKLOADS[name]
        if name == head_name:
            steps, warmup = default_steps(wl, args.steps, args.warmup)
        else:
            steps, warmup = default_steps(wl, None, None)
            if args.steps is not None:
                steps = max(steps, args.steps)
        log(f"[bench] {name}: {steps} steps after {warmup} warm-up")
        # the independent-selection variant differs from its headline only in
        # the inputs: no dense leg (same shapes) and no CPU leg
        variant = wl.direction_scale != 1.0
        records[name] = measure(wl, steps, warmup, args, dev,
                                cpu=not args.no_cpu and not variant,
                                dense=not args.no_dense and not variant,
                                memory=not args.no_memory and not variant)
        log(f"[bench] {name}: {records[name]['value']} query-tokens/s, "
            f"{records[name]['ms_per_step']} ms per step")
    head = records[head_name]
    out = {
        "metric": METRIC, "value": head["value"], "unit": "query-tokens/s", "n_gpus": 1,
        "steps": head["steps"], "warmup": head["warmup"], "ms_per_step": head["ms_per_step"],
        "step_ms": head["step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic", "config": head["config"],
        "roofline": head["roofline"],
        "step_roofline": head["step_roofline"],
        "kernels_us_per_step": head["kernels_us_per_step"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for key in ("indexer_mfma", "projection_mfma", "dense_gqa", "memory", "calls_roofline"):
        if key in head:
            out[key] = head[key]
    if len(records) > 1:
        out["configs"] = {k: v for k, v in records.items() if k != head_name}
    # a counter run's only device copy must be the calibration copy
    if not args.no_peaks and not args.copy_calibration:
        mp_ = measured_peaks(dev)
        out["measured_peaks"] = mp_
        for rec in [out] + list(out.get("configs", {}).values()):
            r = rec["roofline"]
            meas = mp_["hbm_copy_gbs"] if r["unit"] == "GB/s" else mp_["bf16_gemm_tflops"]
            r["frac_of_measured_peak"] = round(r["achieved"] / meas, 4)
            for key in ("indexer_mfma", "projection_mfma"):
                if key in rec:
                    rec[key]["frac_of_measured_peak"] = round(
                        rec[key]["achieved_tflops"] / mp_["bf16_gemm_tflops"], 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
