"""qsa_attn_decode_noalloc (the entry point that allocates nothing: its
split partials and counters live in the library's static scratch) against
qsa_attn_decode with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, outputs bit for bit equal (same
kernels, same split plan) and within tolerance of the oracle."""

import numpy as np
import pytest
import torch

from block_sparse_attention_32_amd import binding as B
from block_sparse_attention_32_amd import pipeline as P
from block_sparse_attention_32_amd import workloads as W

from gpu_helpers import TOL, Problem, f64, sel_rows

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS
CASES = [WL["decode_8x32k"],                                            # 8 rows, 32K context
         WL["decode_8x32k"].replace(name="small", n_ctx=6000, n_seqs=3, seed=17)]  # then smaller


def test_noalloc_decode_matches_workspace_call(gpu):
    for wl in CASES:
        print(f"noalloc {wl.name} seqs={wl.n_seqs} ctx={wl.n_ctx}", flush=True)
        pb = Problem(wl, gpu)
        pb.pool_all()
        st = P.QsaStep(pb.cv, pb.rows, pb.qs.q, pb.qs.q_idx, pb.qs.w, wl.top_k, wl.scale,
                       "decode")
        st.select()
        st.attend()
        got = torch.full_like(st.out, float("nan"))
        B.qsa_attn_decode_noalloc(pb.cv, pb.rows, pb.qs.q, st.sel, st.n_sel, wl.top_k, wl.scale,
                                  got)
        torch.cuda.synchronize()
        assert torch.equal(got, st.out), "differs from qsa_attn_decode"
        _, sel, n = sel_rows(st.sel, st.n_sel)
        out = f64(got)
        for i in range(len(pb.pos_list)):
            want = pb.oracle_attend(i, sel[i, : n[i]])
            err = float(np.abs(out[i] - want).max())
            assert err <= TOL[wl.dtype], f"row {i} err {err}"
