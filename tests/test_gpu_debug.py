"""The debug build (libqsa_debug.so, -DQSA_DEBUG) on the GPU: with valid
inputs it records nothing and computes bit for bit what the release build
computes; invalid device data -- a page id outside the declared pool, a
sequence id or position out of range, a selection length past top_k or a
selected id past the row's blocks -- sets its bit of qsa_debug_take and is
replaced by a value inside the buffers (every case keeps its accesses
inside allocated memory even without the checks)."""

import json
import os
import subprocess
import sys

import pytest
import torch

from block_sparse_attention_32_amd import binding as B

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = os.path.join(ROOT, "tests", "gpu_debug_child.py")


def _child(lib, out):
    env = dict(os.environ, QSA_LIB=lib)
    r = subprocess.run([sys.executable, "-u", CHILD, out], env=env, capture_output=True,
                       text=True, timeout=110)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_debug_build_checks_device_data(gpu, tmp_path):
    if not os.path.exists(B.DEBUG_LIB_PATH):
        pytest.skip("libqsa_debug.so is not built")
    print("debug build: release run", flush=True)
    _child(B.LIB_PATH, str(tmp_path / "release.pt"))
    print("debug build: debug run", flush=True)
    flags = _child(B.DEBUG_LIB_PATH, str(tmp_path / "debug.pt"))
    assert flags["valid"] == 0, flags
    rel = torch.load(tmp_path / "release.pt", weights_only=True)
    dbg = torch.load(tmp_path / "debug.pt", weights_only=True)
    for k in rel:
        assert torch.equal(rel[k], dbg[k]), k
    assert flags["bad_page"] & B.QSA_DEBUG_BAD_PAGE, flags
    assert flags["bad_row"] & B.QSA_DEBUG_BAD_ROW, flags
    assert flags["bad_sel"] & B.QSA_DEBUG_BAD_SEL, flags
    assert flags["bad_sel_prefill"] & B.QSA_DEBUG_BAD_SEL, flags
