"""A decode step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between the
replays, gives bitwise the eager step's outputs, page lists and counts; the
arrival counters of the in-launch merge are zero after every replay; a
replay on queries changed in place matches the eager step on them.

Steps covered: the fused top-k step with the last page refreshed inside the
score launch and several splits merged in the decode launch, the same with
one split, the top-delta step, the fp32-pool (vector-ALU) kernels, and the
metadata in the logical layout (the benchmark's step)."""

import pytest
import torch

import workloads as wl
from _gpu_helpers import geometry
from sparse_long_context_page_amd import DecodeStep, build_meta
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

W = wl.Workload
CASES = [
    (SMALL[2], dict()),                           # bf16, G = 6, 4 splits merged in the launch
    (SMALL[2], dict(n_splits=1)),                 # one split: merged directly
    (SMALL[2], dict(delta=1.0)),                  # top-delta selection
    (SMALL[5], dict()),                           # fp32 pools, 2 splits
    (W("graph_f32_g4_d64_sink", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64,
       ctx_range=(600, 2400), budget_pages=20, n_sink=1, n_local=2, sink_logits=True,
       kv_dtype="f32", seed=51, n_splits=3, dense_splits=4, max_pages=160), dict()),
    (wl.B32_64K, dict()),                         # the benchmark's step
    (SMALL[2], dict(layout="logical", n_splits=1)),  # logical metadata layout, one split
]


def _ids():
    return [f"{w.name}-{'-'.join(f'{k}{v}' for k, v in kw.items()) or 'default'}"
            for w, kw in CASES]


def _snapshot(step, out, lse):
    return {k: v.clone() for k, v in dict(out=out, lse=lse, sel=step.sel,
                                          cnt=step.sel_count).items()}


@pytest.mark.parametrize("case", CASES, ids=_ids())
def test_graph_replays_equal_eager(case):
    w, kw = case
    print(f"case {w.name} {kw}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp, "kv", kw.get("layout", w.meta_layout))
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local,
                      kw.get("n_splits", w.n_splits), w.dense_splits, inp["scale"],
                      delta=kw.get("delta"))
    assert step.fused
    q = inp["q"].clone()

    def run():
        return step.sparse(q, inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                           inp["seq_lens"], inp["sink"], refresh_tail=True)

    out, lse = run()
    torch.cuda.synchronize()
    want = _snapshot(step, out, lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g, lse_g = run()
    torch.cuda.synchronize()

    for i in range(4):
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        step.sel.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(step, out_g, lse_g)
        for k in want:
            assert torch.equal(got[k], want[k]), (w.name, kw, i, k)
        if step.arrivals is not None:
            assert int(step.arrivals.abs().sum()) == 0, (w.name, kw, i)
        # eager work of the program's own between the replays
        torch.randn(1 << 16, device="cuda").sum().item()

    # queries changed in place: the replay follows them
    q.mul_(-0.5)
    out_e, lse_e = run()
    torch.cuda.synchronize()
    want2 = _snapshot(step, out_e, lse_e)
    graph.replay()
    torch.cuda.synchronize()
    got2 = _snapshot(step, out_g, lse_g)
    for k in want2:
        assert torch.equal(got2[k], want2[k]), (w.name, kw, "changed q", k)
