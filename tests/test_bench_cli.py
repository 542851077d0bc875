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
