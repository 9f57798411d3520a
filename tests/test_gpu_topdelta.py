"""Top-delta selection (ps_select_topdelta) through the C ABI against the
fp64 oracle, on inputs whose page bounds are tight (workloads.tighten_pages)
so that the threshold keeps fewer pages than the budget in many units:
selection identical to the oracle's rule applied to the device's own scores,
selection identical outside the ambiguity band to the oracle end to end,
outputs within the rel-L2 gate on the device's page list, and the top-k
selection at an infinite delta or without forced pages. The selection fused
into the decode (ps_select_topdelta_sparse_decode) equals the two launches it
replaces, bit for bit."""

import math

import numpy as np
import pytest
import torch

import oracle as ref
import workloads as wl
from _gpu_helpers import check_unit_outputs, geometry, run_step, unit_host
from sparse_long_context_page_amd import DecodeStep, build_meta, ops

pytestmark = pytest.mark.gpu

W = wl.Workload
# (workload, centre std of the tightened keys, deltas, threshold expected to
# keep fewer pages than the budget in some unit: with one query head per KV
# head the threshold is the head's own and binds often; with larger groups the
# smallest pseudo-max of the group against the largest bound binds rarely)
CASES = [
    (W("td_g1_d128", batch=4, num_q_heads=2, num_kv_heads=2, head_dim=128, ctx_range=(600, 2000),
       budget_pages=24, n_sink=1, n_local=2, seed=41, n_splits=3, dense_splits=4,
       max_pages=130), 2.5, (0.0, 0.5, 2.0), True),
    (W("td_g2_d64_permuted", batch=10, num_q_heads=4, num_kv_heads=2, head_dim=64,
       ctx_range=(300, 1500), budget_pages=16, n_sink=1, n_local=1, permuted_pool=True,
       seed=42, n_splits=2, dense_splits=4, max_pages=100), 3.0, (0.0, 1.0), False),
    (W("td_g6_d128_local4", batch=2, num_q_heads=12, num_kv_heads=2, head_dim=128,
       ctx_range=(1000, 3000), budget_pages=32, n_local=4, seed=43, n_splits=4,
       dense_splits=4, max_pages=200), 2.0, (0.0, 3.0), False),
    (W("td_g1_f32_d64", batch=3, num_q_heads=2, num_kv_heads=2, head_dim=64,
       ctx_range=(200, 900), budget_pages=12, n_sink=2, n_local=1, kv_dtype="f32", seed=44,
       n_splits=2, dense_splits=2, max_pages=60), 2.5, (0.0, 0.5), False),
]


def _inputs(w, spread_std):
    inp = wl.make_inputs(w, device="cuda")
    wl.tighten_pages(inp, center_std=spread_std)
    return inp


def _select(inp, g, scores, budget, n_sink, n_local, delta):
    sel = torch.empty((g.batch, g.num_kv_heads, budget), device="cuda", dtype=torch.int32)
    cnt = torch.empty((g.batch, g.num_kv_heads), device="cuda", dtype=torch.int32)
    ops.ps_select_topdelta(g, inp["q"], inp["k_pool"], inp["page_table"], inp["seq_lens"],
                           scores, budget, n_sink, n_local, inp["scale"], delta, sel, cnt)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy()


def _scores(inp, g):
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    sc = torch.empty((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
    ops.ps_score_pages(g, inp["q"], meta, inp["page_table"], inp["seq_lens"], sc)
    torch.cuda.synchronize()
    return sc


def _oracle_pseudo_max(hu, n, n_sink, n_local, budget):
    forced = sorted(set(range(min(n_sink, n))) | set(range(max(0, n - n_local), n)))
    if budget >= n:
        forced = []
    kf = ref.gather_tokens(hu["k_pool"], hu["kv_dtype"], hu["page_table"], hu["seq_lens"], 0, 0,
                           forced, hu["page_size"])
    return ref.pseudo_max(hu["q"][0].astype(np.float64), kf, hu["scale"])


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_rule_on_device_scores(case):
    """The device's selection equals the oracle's top-delta rule evaluated on
    the device's own scores (only the pseudo-max is the oracle's, in fp64)."""
    w, spread, deltas, binds = case
    inp = _inputs(w, spread)
    g = geometry(inp)
    sc = _scores(inp, g)
    sc_h = sc.cpu().numpy().astype(np.float64)
    fewer = 0
    for delta in deltas:
        sel, cnt = _select(inp, g, sc, w.budget_pages, w.n_sink, w.n_local, delta)
        for b in range(w.batch):
            n = int(inp["n_pages_host"][b])
            for kv in range(w.num_kv_heads):
                hu = unit_host(inp, b, kv)
                mt = _oracle_pseudo_max(hu, n, w.n_sink, w.n_local, w.budget_pages)
                want, _, _, tau = ref.select_pages_topdelta(
                    sc_h[b, kv, :n], n, w.budget_pages, w.n_sink, w.n_local,
                    np.float32(inp["scale"]), mt, delta)
                k = int(cnt[b, kv])
                got = [int(x) for x in sel[b, kv, :k]]
                assert all(int(x) == -1 for x in sel[b, kv, k:])
                if tau is not None:  # pages within 1e-12 of the threshold may go either way
                    near = {p for p in range(n) if
                            abs(float(np.float32(inp["scale"])) * sc_h[b, kv, p] - tau) <=
                            1e-12 * max(abs(tau), 1.0)}
                else:
                    near = set()
                assert set(got) - near == set(int(x) for x in want) - near, (delta, b, kv)
                assert got == sorted(got)
                fewer += k < min(w.budget_pages, n)
    print(f"{w.name}: units keeping fewer pages than the budget: {fewer}")
    assert fewer > 0 or not binds


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_step_end_to_end(case):
    """DecodeStep with delta: selection identical to the oracle's (fp64
    scores) outside the ambiguity band, outputs within the gate on the
    device's page list."""
    w, spread, deltas, _ = case
    inp = _inputs(w, spread)
    g = geometry(inp)
    delta = deltas[0]
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"], delta=delta)
    assert step.fused
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    out, lse = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                           inp["seq_lens"], inp["sink"])
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy().astype(np.float64),
           "lse": lse.cpu().numpy().astype(np.float64)}
    sel, cnt = step.sel.cpu().numpy(), step.sel_count.cpu().numpy()
    for b in range(w.batch):
        for kv in range(w.num_kv_heads):
            hu = unit_host(inp, b, kv)
            r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local, delta=delta)
            n = r["n"]
            mt = _oracle_pseudo_max(hu, n, w.n_sink, w.n_local, w.budget_pages)
            amb = ref.ambiguous_pages_topdelta(r["scores"], n, w.budget_pages, w.n_sink,
                                               w.n_local, hu["scale"], mt, delta,
                                               mag=r["mag"])
            k = int(cnt[b, kv])
            got = set(int(x) for x in sel[b, kv, :k])
            assert got - amb == set(int(x) for x in r["sel"]) - amb, (b, kv)
            check_unit_outputs(res, hu, b, kv, w, w.budget_pages, w.n_sink, w.n_local,
                               sel_dev=sel[b, kv, :k])


def _fused_and_unfused(inp, g, meta, budget, n_sink, n_local, n_splits, delta):
    w = inp["workload"]
    res = []
    for fused in (False, True):
        step = DecodeStep(g, budget, n_sink, n_local, n_splits, w.dense_splits, inp["scale"],
                          fused=fused, delta=delta)
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


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_fused_equals_unfused_bitwise(case):
    """ps_select_topdelta_sparse_decode against ps_select_topdelta then
    ps_sparse_decode (and ps_combine): page lists, counts, partials, merged
    outputs identical, for every delta of the case, with the case's splits
    and with one split (merged in the launch)."""
    w, spread, deltas, binds = case
    inp = _inputs(w, spread)
    g = geometry(inp)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    fewer = 0
    for delta in deltas:
        for ns in (w.n_splits, 1):
            a, b = _fused_and_unfused(inp, g, meta, w.budget_pages, w.n_sink, w.n_local, ns,
                                      delta)
            for k in a:
                assert torch.equal(a[k], b[k]), (w.name, delta, ns, k)
            full = torch.tensor([min(w.budget_pages, int(n)) for n in inp["n_pages_host"]],
                                device="cuda", dtype=torch.int32)[:, None]
            fewer += int((a["cnt"] < full).sum())
    print(f"{w.name}: units keeping fewer pages than the budget: {fewer}")
    assert fewer > 0 or not binds


WIDE_TD = [
    (W("td_wide_g2_d64_units280", batch=70, num_q_heads=8, num_kv_heads=4, head_dim=64,
       ctx_range=(500, 6000), budget_pages=24, n_sink=1, n_local=2, permuted_pool=True,
       max_pages=375, seed=45, n_splits=2, dense_splits=4), 2.5, (0.0, 1.0)),
    (W("td_wide_g1_d128_rows5000", batch=34, num_q_heads=4, num_kv_heads=4, head_dim=128,
       ctx_range=(60000, 80000), budget_pages=64, n_sink=1, n_local=3, max_pages=5000,
       seed=46, n_splits=4, dense_splits=8), 2.5, (0.5,)),
]


@pytest.mark.parametrize("case", WIDE_TD, ids=[c[0].name for c in WIDE_TD])
def test_fused_equals_unfused_wide_grid(case):
    """The same on grids of more than 256 workgroups (4-wavefront decode
    workgroups and their larger selection tiles), with tight bounds."""
    w, spread, deltas = case
    inp = _inputs(w, spread)
    g = geometry(inp)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    for delta in deltas:
        for ns in (w.n_splits, 1):
            a, b = _fused_and_unfused(inp, g, meta, w.budget_pages, w.n_sink, w.n_local, ns,
                                      delta)
            for k in a:
                assert torch.equal(a[k], b[k]), (w.name, delta, ns, k)


@pytest.mark.parametrize("rows", [9000, 20000])
def test_standalone_selection_long_rows(rows):
    """The standalone top-delta selection on rows past the fused decode's limit
    (its register tiles of 32 and 128 pages per lane): the oracle's rule on
    the device's own scores, bit for bit outside 1e-12 of the threshold."""
    w = W(f"td_rows{rows}", batch=2, num_q_heads=1, num_kv_heads=1, head_dim=64,
          ctx_range=(16 * rows - 4000, 16 * rows), budget_pages=48, n_sink=1, n_local=3,
          permuted_pool=True, max_pages=rows, seed=47 + rows % 7)
    inp = _inputs(w, 2.5)
    g = geometry(inp)
    sc = _scores(inp, g)
    sc_h = sc.cpu().numpy().astype(np.float64)
    fewer = 0
    for delta in (0.0, 1.0):
        sel, cnt = _select(inp, g, sc, w.budget_pages, w.n_sink, w.n_local, delta)
        for b in range(w.batch):
            n = int(inp["n_pages_host"][b])
            hu = unit_host(inp, b, 0)
            mt = _oracle_pseudo_max(hu, n, w.n_sink, w.n_local, w.budget_pages)
            want, _, _, tau = ref.select_pages_topdelta(
                sc_h[b, 0, :n], n, w.budget_pages, w.n_sink, w.n_local,
                np.float32(inp["scale"]), mt, delta)
            k = int(cnt[b, 0])
            got = [int(x) for x in sel[b, 0, :k]]
            assert all(int(x) == -1 for x in sel[b, 0, k:])
            near = {p for p in range(n) if tau is not None and
                    abs(float(np.float32(inp["scale"])) * sc_h[b, 0, p] - tau) <=
                    1e-12 * max(abs(tau), 1.0)}
            assert set(got) - near == set(int(x) for x in want) - near, (rows, delta, b)
            assert got == sorted(got)
            fewer += k < min(w.budget_pages, n)
    print(f"rows {rows}: units keeping fewer pages than the budget: {fewer}")


def test_fused_equals_unfused_b32_64k():
    """The same on the 32 x 64k workload in the benchmark's launch
    configuration (delta = 5)."""
    w = wl.B32_64K
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    a, b = _fused_and_unfused(inp, g, meta, w.budget_pages, w.n_sink, w.n_local, w.n_splits,
                              5.0)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("case", CASES[:2], ids=[c[0].name for c in CASES[:2]])
def test_infinite_delta_and_no_forced_pages_are_topk(case):
    w, spread, _, _ = case
    inp = _inputs(w, spread)
    g = geometry(inp)
    sc = _scores(inp, g)
    for budget, ns, nl, delta in ((w.budget_pages, w.n_sink, w.n_local, math.inf),
                                  (w.budget_pages, 0, 0, 0.0), (5, 0, 0, 0.25)):
        a, ca = _select(inp, g, sc, budget, ns, nl, delta)
        sel = torch.empty((g.batch, g.num_kv_heads, budget), device="cuda", dtype=torch.int32)
        cnt = torch.empty((g.batch, g.num_kv_heads), device="cuda", dtype=torch.int32)
        ops.ps_select_topk(g, sc, inp["seq_lens"], budget, ns, nl, sel, cnt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(a, sel.cpu().numpy())
        np.testing.assert_array_equal(ca, cnt.cpu().numpy())


def test_b32_64k_topdelta_keeps_budget():
    """On the 32 x 64k workload (random keys: loose bounds) every page passes
    a threshold of delta = 5, so the selection is the top-k one."""
    w = wl.B32_64K
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    sc = _scores(inp, g)
    a, ca = _select(inp, g, sc, w.budget_pages, w.n_sink, w.n_local, 5.0)
    sel = torch.empty_like(torch.from_numpy(a)).cuda()
    cnt = torch.empty_like(torch.from_numpy(ca)).cuda()
    ops.ps_select_topk(g, sc, inp["seq_lens"], w.budget_pages, w.n_sink, w.n_local, sel, cnt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a, sel.cpu().numpy())


def test_step_with_8bit_metadata():
    """Top-delta selection on scores of 8-bit metadata bounds: the oracle's
    top-delta rule on its 8-bit scores, outside the band; outputs in the gate."""
    w, spread, deltas, _ = CASES[0]
    inp = _inputs(w, spread)
    g = geometry(inp, "fp8")
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"], delta=deltas[0])
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    out, lse = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                           inp["seq_lens"], inp["sink"])
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy().astype(np.float64),
           "lse": lse.cpu().numpy().astype(np.float64)}
    sel, cnt = step.sel.cpu().numpy(), step.sel_count.cpu().numpy()
    fewer = 0
    for b in range(w.batch):
        for kv in range(w.num_kv_heads):
            hu = unit_host(inp, b, kv, meta_format="fp8")
            r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local, delta=deltas[0])
            n = r["n"]
            mt = _oracle_pseudo_max(hu, n, w.n_sink, w.n_local, w.budget_pages)
            amb = ref.ambiguous_pages_topdelta(r["scores"], n, w.budget_pages, w.n_sink,
                                               w.n_local, hu["scale"], mt, deltas[0],
                                               mag=r["mag"])
            k = int(cnt[b, kv])
            assert set(int(x) for x in sel[b, kv, :k]) - amb == \
                set(int(x) for x in r["sel"]) - amb, (b, kv)
            fewer += k < min(w.budget_pages, n)
            check_unit_outputs(res, hu, b, kv, w, w.budget_pages, w.n_sink, w.n_local,
                               sel_dev=sel[b, kv, :k])
    print(f"8-bit metadata, top-delta: units keeping fewer pages than the budget: {fewer}")
