"""bench.py's command line on the host (no GPU work): more than one GPU is
refused with a message, and the workload names it accepts are the seeded
workloads."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_unknown_workload_is_rejected():
    r = _run("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr


def test_help_lists_the_workloads():
    from block_sparse_attention_32_amd import workloads as W
    r = _run("--help")
    assert r.returncode == 0
    for name in ("prefill_1m", "decode_1m", "decode_8x32k", "mtp4_1m"):
        assert name in W.WORKLOADS
        assert name in r.stdout


def _prefill_ctx(W, wl):
    cache = W.make_cache(wl, device="cpu")
    n_chunks = max(1, -(-wl.n_new // (wl.chunk or wl.n_new)))
    chunks = []
    for ci in range(n_chunks):
        seq_id, pos = W.prefill_rows(wl, ci)
        qs = W.make_queries(wl, cache, seq_id, pos, seed=wl.seed + 7919 + ci)
        chunks.append((None, None, None, pos, qs, None))
    return {"cache": cache, "chunks": chunks, "rows": sum(len(c[3]) for c in chunks)}


def test_cpu_baseline_leg_on_small_workloads():
    """The oracle leg of the benchmark on host-resident small workloads:
    decode steps over worker processes, a one-chunk prefill in full, and a
    chunked prefill on the stratified sample (every chunk's edges, every
    t mod 4, rows t <= 2,051, the row after each needle)."""
    sys.path.insert(0, ROOT)
    import bench
    from block_sparse_attention_32_amd import workloads as W

    wl = W.WORKLOADS["decode_8x32k"].replace(n_ctx=3000, n_seqs=3)
    cache = W.make_cache(wl, device="cpu")
    seq_id, pos = W.decode_rows(wl)
    ctx = {"cache": cache, "qs": W.make_queries(wl, cache, seq_id, pos), "pos": pos,
           "rows": len(pos)}
    r = bench.cpu_baseline(wl, ctx, budget_s=1.0)
    assert r["kind"] == "oracle" and r["value"] > 0 and 1 <= r["cores"] <= 3

    wl = W.WORKLOADS["prefill_8k_at_128k"].replace(n_ctx=3000, n_new=64)
    r = bench.cpu_baseline(wl, _prefill_ctx(W, wl), budget_s=1.0)
    assert r["value"] > 0 and "every row" in r["sample"]

    wl = W.WORKLOADS["prefill_1m"].replace(n_new=6144, chunk=2048, n_needles=3)
    ctx = _prefill_ctx(W, wl)
    picks = bench._stratified_prefill_rows(wl, ctx)
    ts = {ctx["chunks"][ci][3][i] for ci, i in picks}
    for ci, c in enumerate(ctx["chunks"]):
        assert set(c[3][:4]) <= ts and set(c[3][-4:]) <= ts
        inner = {c[3][j * len(c[3]) // 15] for j in range(1, 15)}
        assert inner <= ts and len(inner) == 14
    assert {0, 1, 2, 3, 2048, 2051} <= ts
    assert all(4 * (b + 1) in ts for b in ctx["cache"].needles[0])
    r = bench.cpu_baseline(wl, ctx, budget_s=1.0)
    assert r["value"] > 0 and "stratified" in r["sample"]
