"""Soak of the in-launch merge at the 32 x 64k workload: 2000 replays of a
HIP graph holding the fused select + decode launch that merges its own splits
(the last split of each (request, KV head) to finish) followed by ps_combine
over the same partials; after every replay the two outputs and log-sum-exps
are compared bit for bit, and the arrival counters must be zero at the end.
The queries are rescaled in place every 100 replays so that the partials
change. Stops at the first mismatch."""

import pytest
import torch

import workloads as wl
from _gpu_helpers import geometry
from sparse_long_context_page_amd import DecodeStep, build_meta, ops

pytestmark = pytest.mark.gpu

REPLAYS = 2000


def test_in_launch_merge_equals_combine_over_replays():
    w = wl.B32_64K
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp, "kv", w.meta_layout)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"])
    assert step.merge_in_launch and step.n_splits > 1
    q = inp["q"].clone()
    acc, ml = step.partials(step.n_splits)
    out_c = torch.empty_like(step.out)
    lse_c = torch.empty_like(step.lse)
    ops.ps_score_pages(g, q, meta, inp["page_table"], inp["seq_lens"], step.scores)

    def run():
        ops.ps_select_sparse_decode(g, q, inp["k_pool"], inp["v_pool"], inp["page_table"],
                                    inp["seq_lens"], step.scores, w.budget_pages, w.n_sink,
                                    w.n_local, inp["scale"], step.n_splits, step.sel,
                                    step.sel_count, acc, ml, inp["sink"], step.out, step.lse,
                                    arrivals=step.arrivals)
        ops.ps_combine(g, acc, ml, step.n_splits, inp["sink"], out_c, lse_c)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        if i % 100 == 0:
            print(f"[soak] replay {i}", flush=True)
            if i:
                q.mul_(-1.25 if i % 200 else 0.8)  # new partials from here on
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out.view(torch.int32), out_c.view(torch.int32)), i
        assert torch.equal(step.lse.view(torch.int32), lse_c.view(torch.int32)), i
    assert int(step.arrivals.abs().sum()) == 0
