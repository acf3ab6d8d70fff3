"""HIP-graph capture of a decode step: every replay gives the eager step's
results bit for bit (the benchmark times replays of such graphs).  The step
is the benchmarked one -- the indexer with the step's inserts and query-side
rows in its top-k launch, then split attention and its combine -- on a small
c4a workload; between replays the program does eager work of its own."""
import dataclasses

import numpy as np
import pytest
import torch

from tests.gpu_util import host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("qside", [False, True])
def test_decode_step_graph_replays_match_eager(qside):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bench
    import compressed_sparse_long_amd as csl
    from synth import workloads as W
    w = dataclasses.replace(W.c4a_decode(), name="c4a_decode_b4_8k", num_seqs=4, ctx=8192)
    print(f"[gpu] graph replay, {w.name}, qside={qside}", flush=True)
    st = bench.DecodeSetup(w, 1, fused_inserts=True, qside=qside)
    q0 = st.q.clone()
    st.step(0)
    torch.cuda.synchronize()
    assert csl.read_device_error() == 0
    want_topk, want_out = host(st.topk).copy(), host(st.out["c4a"].float()).copy()
    want_q = host(st.q.float()).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step(0)
    for rep in range(4):
        st.topk.fill_(-5)
        st.out["c4a"].zero_()
        if qside:
            st.q.copy_(q0)
        _ = (torch.randn(1 << 20, device="cuda") * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert csl.read_device_error() == 0
        assert np.array_equal(host(st.topk), want_topk), f"replay {rep}: top-k differs"
        assert np.array_equal(host(st.out["c4a"].float()), want_out), f"replay {rep}: attention output differs"
        if qside:
            assert np.array_equal(host(st.q.float()), want_q), f"replay {rep}: q differs"
