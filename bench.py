"""Benchmark of the QSA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic query rows,
with the cache already resident in HBM:
  decode : pool the newest complete block -> indexer scores -> exact top-k
           -> split-K sparse attention (one query row per sequence)
  prefill: pool the chunk's complete blocks -> fused scores + top-k
           -> per-row sparse attention (one chunk of query rows)

Prints one JSON line: query-tokens/s, per-call kernel times from HIP events
on the launch stream, the roofline of the dominant kernel, the dense-GQA
comparison on the same inputs, and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
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

METRIC = "QSA decode/prefill query-tokens/s at 128K & 1M ctx; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


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


def source_hash(*files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_sparse_attention_32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was
    taken on the current kernel source (else null)."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ decode

def run_decode(wl: W.Workload, steps: int, warmup: int, dev):
    from block_sparse_attention_32_amd import pipeline as P
    log(f"[bench] drawing {wl.name} cache on {dev}")
    cache = W.make_cache(wl, device=dev)
    seq_id, pos = W.decode_rows(wl)
    qs = W.make_queries(wl, cache, seq_id, pos, device=dev)
    cv = B.CacheView.from_cache(cache)
    rows = B.QueriesView(qs.seq_id, qs.pos, max(pos))
    n_blocks = wl.total_len // 4
    P.pool_all(cv, wl.n_seqs, n_blocks, dev)               # set-up, untimed
    step = P.QsaStep(cv, rows, qs.q, qs.q_idx, qs.w, wl.top_k, wl.scale, "decode")
    max_n = max(pos) // 4
    scores = torch.empty((rows.n_rows, max_n), dtype=torch.float32, device=dev)
    newest = torch.full((wl.n_seqs,), n_blocks - 1, dtype=torch.int32, device=dev)

    def one(timer=None):
        call = timer.wrap if timer else (lambda name, fn, *a, **k: fn(*a, **k))
        call("pool", B.qsa_pool_blocks, cv, newest, 1)
        call("scores", B.qsa_index_scores, cv, rows, qs.q_idx, qs.w, scores)
        call("topk", step.select, scores)
        call("attn", step.attend)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer = Timer()
    for _ in range(steps):
        one(timer)
    torch.cuda.synchronize()
    kern = timer.avg_us()

    # dense GQA flash-decode on the same inputs (comparison baseline)
    dense = P.DenseStep(cv, rows, qs.q, wl.scale, "decode")
    for _ in range(max(2, warmup // 2)):
        dense.run()
    torch.cuda.synchronize()
    n_dense = max(5, steps // 4)
    t1 = time.perf_counter()
    for _ in range(n_dense):
        dense.run()
    torch.cuda.synchronize()
    dense_ms = 1e3 * (time.perf_counter() - t1) / n_dense

    n_sel = step.n_sel.cpu().numpy()
    n_tok = int(sum(4 * int(n) + p % 4 + 1 for n, p in zip(n_sel, pos)))
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        "scores": {"bytes": sum(p // 4 for p in pos) * wl.di * esz, "bound": "hbm"},
        "attn": {"bytes": n_tok * wl.hkv * wl.d * esz * 2, "bound": "hbm"},
        "topk": {"bytes": sum(p // 4 for p in pos) * 4, "bound": "hbm"},
        "pool": {"bytes": wl.n_seqs * 5 * wl.di * esz, "bound": "hbm"},
    }
    kernels = {"scores": "scores_kernel", "attn": "attn_kernel", "topk": "topk_pass_a+b",
               "pool": "pool_kernel"}
    files = {"scores": ("index.hip", "index.hpp", "common.hpp"),
             "attn": ("attention.hip", "attention.hpp", "common.hpp"),
             "topk": ("index.hip", "index.hpp", "select.hpp", "common.hpp"),
             "pool": ("index.hip", "index.hpp", "common.hpp")}
    ctx = dict(rows=rows.n_rows, sel=(step, cache, qs, pos))
    return wall, kern, work, kernels, files, dense_ms, ctx


# ------------------------------------------------------------------ prefill

def run_prefill(wl: W.Workload, steps: int, warmup: int, dev, dense_too: bool = True):
    """One step = the whole prefill of wl: every chunk of query rows in
    order (pool the chunk's new blocks -> fused scores + top-k -> per-row
    sparse attention).  The existing context (if any) is pooled at set-up."""
    from block_sparse_attention_32_amd import pipeline as P
    log(f"[bench] drawing {wl.name} cache on {dev}")
    cache = W.make_cache(wl, device=dev)
    cv = B.CacheView.from_cache(cache)
    n_chunks = max(1, -(-wl.n_new // (wl.chunk or wl.n_new)))
    chunks = []
    for ci in range(n_chunks):
        seq_id, pos = W.prefill_rows(wl, ci)
        qs = W.make_queries(wl, cache, seq_id, pos, device=dev, seed=wl.seed + 7919 + ci)
        rows = B.QueriesView(qs.seq_id, qs.pos, max(pos))
        st = P.QsaStep(cv, rows, qs.q, qs.q_idx, qs.w, wl.top_k, wl.scale, "prefill")
        b0 = pos[0] // 4
        begin = torch.full((1,), b0, dtype=torch.int32, device=dev)
        chunks.append((st, begin, (pos[-1] + 1) // 4 - b0, pos))
    if wl.n_ctx:
        P.pool_all(cv, 1, wl.n_ctx // 4, dev)               # set-up, untimed

    def one(timer=None):
        call = timer.wrap if timer else (lambda name, fn, *a, **k: fn(*a, **k))
        for st, begin, nb, _ in chunks:
            call("pool", B.qsa_pool_blocks, cv, begin, nb)
            call("topk", st.select)
            call("attn", st.attend)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer = Timer()
    one(timer)
    torch.cuda.synchronize()
    kern = {k: v * len(chunks) for k, v in timer.avg_us().items()}   # per step
    rows_total = sum(len(c[3]) for c in chunks)
    n_tok = 0
    cand = 0
    for st, _, _, pos in chunks:
        ns = st.n_sel.cpu().numpy().astype(np.int64)
        p_ = np.asarray(pos, dtype=np.int64)
        n_tok += int((4 * ns + p_ % 4 + 1).sum())
        cand += int((p_ // 4).sum())
    esz = 2 if wl.dtype == "bf16" else 4
    work = {
        "attn": {"bytes": n_tok * wl.hkv * wl.d * esz * 2, "flops": 4 * wl.hq * wl.d * n_tok,
                 "bound": "hbm"},
        "topk": {"flops": 2 * wl.hi * wl.di * cand, "bound": "alu"},
        "pool": {"bytes": (wl.n_new // 4) * 5 * wl.di * esz, "bound": "hbm"},
    }
    return wall, kern, work, rows_total, chunks, cache


# ------------------------------------------------------------------ CPU oracle

def cpu_baseline_decode(wl, ctx, budget_s=12.0):
    """The oracle's decode step (pool the newest block, score every candidate,
    select, attend) on rank 0's host cores, repeated for about budget_s."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    step, cache, qs, pos = ctx["sel"]
    log("[bench] cpu oracle: copying the cache to host")
    seqs = []
    for s in range(wl.n_seqs):
        k, v, kidx = W.seq_view(cache, s)
        seqs.append((k.float().cpu().numpy(), v.float().cpu().numpy(),
                     kidx.double().cpu().numpy()))
    q = qs.q.double().cpu().numpy()
    q_idx = qs.q_idx.double().cpu().numpy()
    w = qs.w.double().cpu().numpy()
    kbars = [O.pool_blocks(kidx, wl.dtype) for _, _, kidx in seqs]   # set-up, untimed
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            for i, t in enumerate(pos):
                k, v, kidx = seqs[i]
                nb = (t + 1) // 4
                kbars[i][nb - 1:nb] = O.pool_blocks(kidx[: 4 * nb], wl.dtype, nb - 1, nb)
                O.qsa_row(k, v, kbars[i], q[i], q_idx[i], w[i], t, wl.top_k, wl.scale)
                done += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return {"value": done / el, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} decode query rows of {wl.name} (full candidate range each), "
                      f"{el:.1f} s, numpy float64 single-threaded"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_1m", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
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
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if wl.mode != "decode":
        wall, kern, work, rows_total, chunks, cache = run_prefill(wl, args.steps, args.warmup, dev)
        ms = 1e3 * wall / args.steps
        out = {
            "metric": METRIC, "value": round(rows_total / (wall / args.steps), 1),
            "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
            "config": {"workload": wl.name, "context": wl.n_ctx, "new_tokens": wl.n_new,
                       "chunk": wl.chunk or wl.n_new, "hq": wl.hq, "hkv": wl.hkv,
                       "head_dim": wl.d, "idx_heads": wl.hi, "idx_dim": wl.di,
                       "top_k": wl.top_k, "page_size": wl.page_size,
                       "parallelism": "single-gpu"},
            "kernels_us": {k: round(v, 1) for k, v in kern.items()},
            "work": work,
        }
        print(json.dumps(out), flush=True)
        return
    wall, kern, work, kernels, files, dense_ms, ctx = run_decode(wl, args.steps, args.warmup, dev)
    ms = 1e3 * wall / args.steps
    value = ctx["rows"] / (wall / args.steps)
    dom = max(kern, key=kern.get)
    wk = work[dom]
    src_hash = source_hash(*files[dom])
    achieved = wk["bytes"] / (kern[dom] * 1e-6) / 1e9
    roof = {"kernel": kernels[dom], "bound": wk["bound"], "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(kernels[dom], wl.name, src_hash),
            "algorithmic_bytes": wk["bytes"], "avg_us": round(kern[dom], 2),
            "source_hash": src_hash}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_decode(wl, ctx)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "n_seqs": wl.n_seqs, "context": wl.n_ctx,
                   "query_rows": ctx["rows"], "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d,
                   "idx_heads": wl.hi, "idx_dim": wl.di, "top_k": wl.top_k,
                   "page_size": wl.page_size, "parallelism": "single-gpu"},
        "roofline": roof,
        "kernels_us": {k: round(v, 2) for k, v in kern.items()},
        "kernel_sum_us": round(sum(kern.values()), 2),
        "dense_gqa": {"ms_per_step": round(dense_ms, 4),
                      "speedup_sparse_over_dense": round(dense_ms / ms, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
