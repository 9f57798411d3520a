"""The fused selection + sparse decode (ps_select_sparse_decode) against the
two launches it replaces (ps_select_topk then ps_sparse_decode): the page
list, the counts, the split partials and the merged outputs are bitwise
identical, on the small workloads (bf16 and fp32 pools, several splits,
ragged tails, sink and local pages, budgets that cover every page of short
requests), on fp32 pools with longer rows (the selection's larger register
tiles) and on the 32 x 64k workload in the benchmark's launch
configuration; with several splits the merge made in the launch by the last
split of each (request, KV head) equals ps_combine's, bit for bit."""

import pytest
import torch

import workloads as wl
from _gpu_helpers import geometry
from sparse_long_context_page_amd import DecodeStep, build_meta, ops
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

# fp32 pools with rows of 563 and 2500 pages (selection tiles of 8 and 32
# pages per lane in the 4-wavefront fp32 decode)
F32_LONG = [
    wl.Workload("f32_g4_d128_sink_local_rows563", batch=3, num_q_heads=8, num_kv_heads=2,
                head_dim=128, ctx_range=(2000, 9000), budget_pages=24, n_sink=1, n_local=3,
                needles=3, sink_logits=True, permuted_pool=True, max_pages=563,
                kv_dtype="f32", seed=31, n_splits=3, dense_splits=8),
    wl.Workload("f32_g6_d64_rows2500", batch=2, num_q_heads=12, num_kv_heads=2, head_dim=64,
                ctx_range=(30000, 40000), budget_pages=40, n_local=2, needles=4,
                max_pages=2500, kv_dtype="f32", seed=32, n_splits=4, dense_splits=8),
]
# bf16 pools on grids of more than 256 workgroups (4-wavefront decode
# workgroups), rows of 375 and 5000 pages (selection tiles of 16 and 32 pages
# per lane)
WIDE = [
    wl.Workload("wide_g2_d64_units280", batch=70, num_q_heads=8, num_kv_heads=4, head_dim=64,
                ctx_range=(500, 6000), budget_pages=24, n_sink=1, n_local=2, needles=2,
                permuted_pool=True, max_pages=375, seed=33, n_splits=2, dense_splits=4),
    wl.Workload("wide_g6_d128_rows5000", batch=34, num_q_heads=12, num_kv_heads=2,
                head_dim=128, ctx_range=(60000, 80000), budget_pages=64, n_local=4, needles=4,
                max_pages=5000, seed=34, n_splits=4, dense_splits=8),
]
CASES = SMALL + F32_LONG + WIDE + [wl.B32_64K]


def _both(inp, budget=None, n_sink=None, n_local=None, n_splits=None):
    w = inp["workload"]
    g = geometry(inp)
    budget = w.budget_pages if budget is None else budget
    kw = dict(n_sink=w.n_sink if n_sink is None else n_sink,
              n_local=w.n_local if n_local is None else n_local,
              n_splits=w.n_splits if n_splits is None else n_splits,
              dense_splits=w.dense_splits, scale=inp["scale"])
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    res = []
    for fused in (False, True):
        step = DecodeStep(g, budget, fused=fused, **kw)
        assert step.fused == fused
        step.sel.fill_(-7)
        step.sel_count.fill_(-7)
        out, lse = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                               inp["seq_lens"], inp["sink"])
        acc, ml = step.partials(step.n_splits)
        torch.cuda.synchronize()
        got = dict(sel=step.sel, cnt=step.sel_count, out=out, lse=lse)
        if step.n_splits > 1:  # with one split the fused launch writes no partials
            got.update(acc=acc, ml=ml)
        res.append({k: v.clone() for k, v in got.items()})
    return res


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_fused_equals_unfused_bitwise(w):
    inp = wl.make_inputs(w, device="cuda")
    configs = [dict()]
    if w.batch * w.num_kv_heads <= 16:  # more budgets and splits on the small ones
        configs += [dict(budget=3, n_sink=1, n_local=1, n_splits=2),
                    dict(budget=1, n_sink=0, n_local=0, n_splits=1),
                    dict(budget=64, n_sink=2, n_local=3, n_splits=7)]
    for cfg in configs:
        a, b = _both(inp, **cfg)
        for k in a:
            assert torch.equal(a[k], b[k]), (w.name, cfg, k)


def test_fused_without_page_list_output():
    w = SMALL[2]
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    a, _ = _both(inp)
    assert w.n_splits > 1
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"])
    ops.ps_score_pages(g, inp["q"], meta, inp["page_table"], inp["seq_lens"], step.scores)
    acc, ml = step.partials(step.n_splits)
    ops.ps_select_sparse_decode(g, inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                inp["seq_lens"], step.scores, w.budget_pages, w.n_sink,
                                w.n_local, inp["scale"], step.n_splits, None, None, acc, ml)
    torch.cuda.synchronize()
    assert torch.equal(acc, a["acc"]) and torch.equal(ml, a["ml"])


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_fused_one_split_merged_output_bitwise(w):
    """With one split the fused launch also merges (sink in the denominator):
    equal, bit for bit, to the unfused one-split decode followed by
    ps_combine, page lists included."""
    inp = wl.make_inputs(w, device="cuda")
    a, b = _both(inp, n_splits=1)
    for k in ("sel", "cnt", "out", "lse"):
        assert torch.equal(a[k], b[k]), (w.name, k)
    if inp["sink"] is not None:  # and without the sink
        g = geometry(inp)
        meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
        step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, 1, w.dense_splits,
                          inp["scale"], fused=False)
        want, _ = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                              inp["seq_lens"], None)
        want = want.clone()
        step2 = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, 1, w.dense_splits,
                           inp["scale"], fused=True)
        got, _ = step2.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                              inp["seq_lens"], None)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


# several splits need a budget of two pages or more
MULTI = [w for w in CASES if w.budget_pages >= 2]


@pytest.mark.parametrize("w", MULTI, ids=[w.name for w in MULTI])
def test_in_launch_merge_of_several_splits_bitwise(w):
    """With several splits and a merged output, the last split of each
    (request, KV head) to finish merges them in the launch: outputs and lse
    equal, bit for bit, to ps_combine over the same partials (with and
    without the sink, and without lse); page lists and partials unchanged;
    the arrival counters are zero after every launch, and the next launches,
    on other queries, reuse them and are exact again."""
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    ns = max(2, min(w.n_splits, w.budget_pages))
    mk = dict(budget_pages=w.budget_pages, n_sink=w.n_sink, n_local=w.n_local, n_splits=ns,
              dense_splits=w.dense_splits, scale=inp["scale"])
    merged = DecodeStep(g, **mk)
    plain = DecodeStep(g, **mk, merge_in_launch=False)
    assert merged.merge_in_launch and plain.fused and not plain.merge_in_launch
    queries = [inp["q"], -inp["q"], inp["q"] * 0.5]
    sinks = [inp["sink"], None, inp["sink"]]
    for i, (q, sink) in enumerate(zip(queries, sinks)):
        merged.out.fill_(float("nan"))
        merged.lse.fill_(float("nan"))
        got = merged.sparse(q, inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                            inp["seq_lens"], sink)
        want = plain.sparse(q, inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                            inp["seq_lens"], sink)
        torch.cuda.synchronize()
        for a, b, k in zip(got, want, ("out", "lse")):
            assert torch.equal(a, b), (w.name, i, k)
        for a, b in zip(merged.partials(ns), plain.partials(ns)):
            assert torch.equal(a, b), (w.name, i)
        assert torch.equal(merged.sel, plain.sel) and torch.equal(merged.sel_count,
                                                                   plain.sel_count)
        assert int(merged.arrivals.abs().sum()) == 0, (w.name, i)
    # without lse: the same output
    out = torch.full_like(merged.out, float("nan"))
    acc, ml = merged.partials(ns)
    ops.ps_select_sparse_decode(g, queries[-1], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                inp["seq_lens"], merged.scores, w.budget_pages, w.n_sink,
                                w.n_local, inp["scale"], ns, None, None, acc, ml, sinks[-1],
                                out, None, arrivals=merged.arrivals)
    torch.cuda.synchronize()
    assert torch.equal(out, plain.out)
    assert int(merged.arrivals.abs().sum()) == 0


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_refresh_score_equals_meta_then_score_bitwise(w):
    """ps_refresh_score_pages on metadata whose last pages are stale equals
    the full metadata build followed by ps_score_pages, bit for bit (the
    refreshed last pages included)."""
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    full = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    want = torch.empty((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
    ops.ps_score_pages(g, inp["q"], full, inp["page_table"], inp["seq_lens"], want)
    stale = full.clone()
    tails = [int(inp["page_table"][b, int(n) - 1]) for b, n in enumerate(inp["n_pages_host"])]
    stale[tails] = 3.0  # what the pages held before the last token was appended
    got = torch.full_like(want, float("nan"))
    ops.ps_refresh_score_pages(g, inp["q"], inp["k_pool"], stale, inp["page_table"],
                               inp["seq_lens"], got)
    torch.cuda.synchronize()
    assert torch.equal(stale, full)
    for b, n in enumerate(inp["n_pages_host"]):
        assert torch.equal(got[b, :, :int(n)], want[b, :, :int(n)]), (w.name, b)


def test_step_with_tail_refresh_fused_equals_unfused():
    w = SMALL[4]  # sink page, local pages, permuted pool, lengths from 1 token
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    tail = torch.tensor([int(n) - 1 for n in inp["n_pages_host"]], device="cuda",
                        dtype=torch.int32)
    outs = []
    for fused in (False, True):
        meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
        meta[[int(inp["page_table"][b, int(n) - 1]) for b, n in
              enumerate(inp["n_pages_host"])]] = -2.0
        step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                          inp["scale"], fused=fused)
        if not fused:  # the tail pages rebuilt by a launch of their own, then four more
            step.refresh_tail_meta(inp["k_pool"], inp["page_table"], inp["seq_lens"], tail, meta)
        out, lse = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                               inp["seq_lens"], inp["sink"], refresh_tail=fused)
        torch.cuda.synchronize()
        outs.append((meta.clone(), step.sel.clone(), out.clone(), lse.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
