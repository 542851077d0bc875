"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pin tests catch every one of them."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "qsa_oracle.py")

MUTATIONS = {
    "pool_drops_last_row": ("rows = kidx[block * b: block * b + block]",
                            "rows = kidx[block * b: block * b + block - 1]"),
    "pool_sum_not_mean": ("rows.sum(axis=0) / block", "rows.sum(axis=0)"),
    "pool_ignores_block_size": ("rows = kidx[block * b: block * b + block]",
                                "rows = kidx[BLOCK * b: BLOCK * b + BLOCK]"),
    "pool_divides_by_four": ("rows.sum(axis=0) / block", "rows.sum(axis=0) / BLOCK"),
    "token_set_four_tokens": ("toks = [block * int(b) + i for b in sel for i in range(block)]\n    toks += list(range(block * own_block(t, block), t + 1))",
                              "toks = [block * int(b) + i for b in sel for i in range(BLOCK)]\n    toks += list(range(block * own_block(t, block), t + 1))"),
    "own_block_default_size": ("    return own_block(t, block)\n", "    return own_block(t)\n"),
    "relu_sign": ("np.maximum(dots, 0.0)", "np.maximum(-dots, 0.0)"),
    "no_relu": ("np.maximum(dots, 0.0)", "dots"),
    "weight_index": ("s += w[h] *", "s += w[0] *"),
    "tie_to_higher_id": ("order = np.lexsort((ids, -scores))",
                         "order = np.lexsort((-ids, -scores))"),
    "select_lowest": ("order = np.lexsort((ids, -scores))",
                      "order = np.lexsort((ids, scores))"),
    "own_block_cut": ("toks += list(range(block * own_block(t, block), t + 1))",
                      "toks += list(range(block * own_block(t, block), t))"),
    "shared_tail_from_own_block": ("range(block * own_block(t_sel, block), t + 1)",
                                   "range(block * own_block(t, block), t + 1)"),
    "shared_tail_cut": ("range(block * own_block(t_sel, block), t + 1)",
                        "range(block * own_block(t_sel, block), t)"),
    "project_head_order": ("return q.reshape(x.shape[0], n_heads, -1), k, w",
                           "return q.reshape(x.shape[0], -1, n_heads).transpose(0, 2, 1), k, w"),
    "project_key_from_query_weights": ("k = round_to_storage(x @ np.asarray(wk, dtype=np.float64).T, dtype)",
                                       "k = round_to_storage(x @ np.asarray(wq, dtype=np.float64)[: len(wk)].T, dtype)"),
    "own_block_competes": ("return own_block(t, block)\n", "return own_block(t, block) + 1\n"),
    "gqa_interleaved": ("return hq // (n_q_heads // n_kv_heads)",
                        "return hq % n_kv_heads"),
    "softmax_no_scale": ("z = scale * (kk @ q[hq])", "z = (kk @ q[hq])"),
    "bf16_spacing": ("spacing = np.ldexp(1.0, e - 8)", "spacing = np.ldexp(1.0, e - 9)"),
    "bf16_truncates": ("return np.rint(x / spacing) * spacing",
                       "return np.trunc(x / spacing) * spacing"),
    "f32_no_rounding": ("return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)",
                        "return np.asarray(x, dtype=np.float64)"),
    "f32_truncates": ("return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)",
                      "return (lambda m, e: np.ldexp(np.trunc(np.ldexp(m, 24)), e - 24))"
                      "(*np.frexp(np.asarray(x, dtype=np.float64)))"),
    "mask_wrong_head": ("z = scale * (q[:, hq, :] @ k[:, hk, :].T)",
                        "z = scale * (q[:, hq, :] @ k[:, hq % k.shape[1], :].T)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(ORACLE).read()
    assert src.count(before) >= 1, "mutation target vanished from the oracle"
    dst = tmp_path / "repo"
    os.makedirs(dst / "block_sparse_attention_32_amd")
    shutil.copytree(os.path.join(ROOT, "oracle"), dst / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), dst / "tests",
                    ignore=shutil.ignore_patterns("__pycache__"))
    for f in ("__init__.py", "workloads.py"):
        shutil.copy(os.path.join(ROOT, "block_sparse_attention_32_amd", f),
                    dst / "block_sparse_attention_32_amd" / f)
    (dst / "oracle" / "qsa_oracle.py").write_text(src.replace(before, after))
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         "tests/test_oracle_pins.py", "tests/test_workloads.py"],
        cwd=dst, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin"
