"""A decode step (fused pooling + top-k, then split-K attention) captured
once in a HIP graph and replayed: every replay, with eager steps and
synchronisations between the replays, gives the eager step's selection and
output bit for bit (the library's calls enqueue kernels only -- no memset
nodes -- and leave their workspace counters at zero)."""

import pytest
import torch

from block_sparse_attention_32_amd import binding as B
from block_sparse_attention_32_amd import pipeline as P
from block_sparse_attention_32_amd import workloads as W

from gpu_helpers import Problem

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode_8x32k", "decode_1m"])
def test_decode_step_graph_replays_match_eager(gpu, name):
    print(f"graph replay {name}", flush=True)
    wl = W.WORKLOADS[name]
    pb = Problem(wl, gpu)
    pb.pool_all()
    st = P.QsaStep(pb.cv, pb.rows, pb.qs.q, pb.qs.q_idx, pb.qs.w, wl.top_k, wl.scale, "decode")

    def step():
        st.select_pooling_newest()
        st.attend()

    step()
    torch.cuda.synchronize()
    want = (st.sel.clone(), st.n_sel.clone(), st.out.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (st.sel, st.n_sel):
            t.fill_(-9)
        st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (st.sel, st.n_sel, st.out)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        step()                      # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip((st.sel, st.n_sel, st.out), want):
            assert torch.equal(a, b), f"eager step after replay {rep} differs"
