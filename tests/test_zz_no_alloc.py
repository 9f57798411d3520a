"""The decode entry point without allocation (ps_select_sparse_decode_noalloc)
against the fused decode with caller workspace (ps_select_sparse_decode with
out and arrivals), through the C ABI: bitwise equal page lists, counts,
outputs and log-sum-exps, on two calls in a row of which the second has a
smaller input, run on one stream, and again under HIP graph capture with
several replays, each checked against the eager result."""

import numpy as np
import pytest
import torch

import workloads as wl
from _gpu_helpers import geometry
from sparse_long_context_page_amd import build_meta, ops

pytestmark = pytest.mark.gpu

BIG = wl.Workload("noalloc_big", batch=6, num_q_heads=12, num_kv_heads=2, head_dim=128,
                  ctx_range=(900, 4000), budget_pages=40, n_local=2, needles=2,
                  permuted_pool=True, seed=515, n_splits=4)
SMALL = wl.Workload("noalloc_small", batch=3, num_q_heads=8, num_kv_heads=1, head_dim=64,
                    ctx_range=(100, 1200), budget_pages=20, n_sink=1, sink_logits=True,
                    seed=516, n_splits=3)
ONE_SPLIT = SMALL.replace(name="noalloc_one_split", n_splits=1, seed=517)


def _prepared(w):
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    scores = torch.empty((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
    ops.ps_score_pages(g, inp["q"], meta, inp["page_table"], inp["seq_lens"], scores)
    return inp, g, scores


def _outputs(g, w):
    b, hq, hkv, d = g.batch, g.num_q_heads, g.num_kv_heads, g.head_dim
    return (torch.full((b, hkv, w.budget_pages), -9, device="cuda", dtype=torch.int32),
            torch.full((b, hkv), -9, device="cuda", dtype=torch.int32),
            torch.full((b, hq, d), float("nan"), device="cuda"),
            torch.full((b, hq), float("nan"), device="cuda"))


def _with_workspace(inp, g, scores, w):
    sel, cnt, out, lse = _outputs(g, w)
    ns = w.n_splits
    acc = torch.empty((g.batch, g.num_q_heads, ns, g.head_dim), device="cuda")
    ml = torch.empty((g.batch, g.num_q_heads, ns, 2), device="cuda")
    arr = torch.zeros((g.batch, g.num_kv_heads), device="cuda", dtype=torch.int32)
    ops.ps_select_sparse_decode(g, inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                inp["seq_lens"], scores, w.budget_pages, w.n_sink, w.n_local,
                                inp["scale"], ns, sel, cnt, acc if ns > 1 else None,
                                ml if ns > 1 else None, inp["sink"], out, lse,
                                arrivals=arr if ns > 1 else None)
    torch.cuda.synchronize()
    assert int(arr.abs().sum()) == 0
    return sel, cnt, out, lse


def _noalloc(inp, g, scores, w, bufs=None):
    sel, cnt, out, lse = _outputs(g, w) if bufs is None else bufs
    ops.ps_select_sparse_decode_noalloc(g, inp["q"], inp["k_pool"], inp["v_pool"],
                                        inp["page_table"], inp["seq_lens"], scores,
                                        w.budget_pages, w.n_sink, w.n_local, inp["scale"],
                                        w.n_splits, sel, cnt, inp["sink"], out, lse)
    return sel, cnt, out, lse


def _equal(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_two_calls_in_a_row_second_smaller():
    runs = [_prepared(w) + (w,) for w in (BIG, SMALL, ONE_SPLIT)]
    want = [_with_workspace(*r) for r in runs]
    got = []
    for r in runs:  # back to back on one stream: big, then smaller, then one split
        print(f"[noalloc] {r[3].name}", flush=True)
        got.append(_noalloc(*r))
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        _equal(a, b)
        assert not torch.isnan(a[2]).any()


def test_replays_of_a_captured_call():
    inp, g, scores, w = _prepared(BIG) + (BIG,)
    want = _with_workspace(inp, g, scores, w)
    bufs = _outputs(g, w)
    _noalloc(inp, g, scores, w, bufs)  # warm-up outside the capture
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        _noalloc(inp, g, scores, w, bufs)
    for i in range(4):
        for t in bufs:
            t.fill_(-3) if t.dtype == torch.int32 else t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        print(f"[noalloc] replay {i}", flush=True)
        _equal(bufs, want)
        # eager work between the replays
        _noalloc(*_prepared(SMALL), SMALL)
        torch.cuda.synchronize()


def test_rejects_a_call_beyond_the_workspace():
    w = wl.Workload("noalloc_too_big", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=64,
                    context=256, budget_pages=16, seed=518, n_splits=8)
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    scores = torch.zeros((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
    sel, cnt, out, lse = _outputs(g, w)
    with pytest.raises(ops._lib.PsError) as e:
        _noalloc(inp, g, scores, w, (sel, cnt, out, lse))
    assert e.value.status == ops._lib.PS_ERR_WORKSPACE
    assert int((sel == -9).sum()) == sel.numel()  # nothing enqueued
