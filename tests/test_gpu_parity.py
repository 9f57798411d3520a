"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Small workloads (the oracle finishes in seconds) span several score, select
and decode tiles, ragged tails, partial last pages, permuted pools, every
supported group size and both head dims and dtypes. Every stage is checked on
its own (metadata bit-exact; scores within SCORE_REL of fp64; selection
bit-exact on given scores; decode and merge on the oracle's page list) and
end to end (selection identical outside the ambiguity band; outputs within
the rel-L2 gate).
"""

import math

import numpy as np
import pytest
import torch

import oracle as ref
import workloads as wl
from _gpu_helpers import (SCORE_REL, check_meta_unit, check_selection, check_unit_outputs,
                          gate, geometry, rel_l2, run_step, score_rel_err, unit_host)
from sparse_long_context_page_amd import DecodeStep, build_meta, ops

pytestmark = pytest.mark.gpu

W = wl.Workload
SMALL = [
    wl.TINY,
    wl.TINY_DENSE,
    W("gqa6_d128_ragged_local", batch=3, num_q_heads=12, num_kv_heads=2, head_dim=128,
      ctx_range=(900, 3000), budget_pages=16, n_local=4, needles=2, permuted_pool=True,
      max_pages=200, seed=21, n_splits=4, dense_splits=8),
    W("gqa8_d64_sink", batch=2, num_q_heads=16, num_kv_heads=2, head_dim=64,
      ctx_range=(700, 1100), budget_pages=8, sink_logits=True, seed=22, n_splits=3,
      dense_splits=5),
    W("gqa7_d128_sinkpage_local", batch=4, num_q_heads=14, num_kv_heads=2, head_dim=128,
      ctx_range=(1, 2500), budget_pages=12, n_sink=1, n_local=2, needles=1,
      permuted_pool=True, max_pages=160, seed=23, n_splits=5, dense_splits=7),
    W("g1_f32_d128", batch=2, num_q_heads=2, num_kv_heads=2, head_dim=128, ctx_range=(300, 520),
      budget_pages=5, kv_dtype="f32", seed=24, n_splits=2, dense_splits=3),
    W("g3_d64_page_aligned", batch=2, num_q_heads=6, num_kv_heads=2, head_dim=64, context=1024,
      budget_pages=10, n_sink=2, n_local=2, needles=2, seed=25, n_splits=10, dense_splits=16),
    W("g2_f32_d64_tiny_contexts", batch=5, num_q_heads=4, num_kv_heads=2, head_dim=64,
      ctx_range=(1, 40), budget_pages=2, kv_dtype="f32", seed=26, n_splits=2, dense_splits=2),
    W("g5_d128_b1_budget1", batch=1, num_q_heads=5, num_kv_heads=1, head_dim=128, context=777,
      budget_pages=1, seed=27, n_splits=1, dense_splits=4),
    W("g4_d64_edge_lengths", batch=6, num_q_heads=4, num_kv_heads=1, head_dim=64,
      lengths=(1, 16, 17, 31, 32, 33), budget_pages=2, n_local=1, seed=28, n_splits=2,
      dense_splits=3),
]


@pytest.fixture(scope="module")
def cases():
    out = {}
    for w in SMALL:
        inp = wl.make_inputs(w, device="cuda")
        res = run_step(inp)
        units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
        out[w.name] = (w, inp, res, {u: unit_host(inp, *u) for u in units})
    return out


def _ids(ws):
    return [w.name for w in ws]


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_meta_bit_exact(cases, w):
    _, inp, res, hosts = cases[w.name]
    for (b, g), hu in hosts.items():
        check_meta_unit(inp, res["meta"], hu, b, g)


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_scores_match_fp64(cases, w):
    _, inp, res, hosts = cases[w.name]
    worst = 0.0
    for (b, g), hu in hosts.items():
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
        n = r["n"]
        worst = max(worst, score_rel_err(res["scores"][b, g, :n].astype(np.float64),
                                         r["scores"], mag=r["mag"]))
    print(f"{w.name}: max score rel err {worst:.3e}")
    assert worst <= SCORE_REL


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_selection_end_to_end(cases, w):
    _, inp, res, hosts = cases[w.name]
    n_amb = 0
    for (b, g), hu in hosts.items():
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
        a, _ = check_selection(res["sel"][b, g], res["sel_count"][b, g], r["scores"], r["n"],
                               w.budget_pages, w.n_sink, w.n_local, mag=r["mag"])
        n_amb += a
    print(f"{w.name}: ambiguous pages {n_amb}")


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_outputs_end_to_end(cases, w):
    _, inp, res, hosts = cases[w.name]
    worst = 0.0
    for (b, g), hu in hosts.items():
        k = int(res["sel_count"][b, g])
        e, _ = check_unit_outputs(res, hu, b, g, w, w.budget_pages, w.n_sink, w.n_local,
                                  sel_dev=res["sel"][b, g, :k])
        worst = max(worst, e)
    print(f"{w.name}: max rel-L2 {worst:.3e} (gate {gate(w)})")


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_select_on_given_scores_bit_exact(w):
    """The select kernel on fixed fp32 scores (including many exact ties)
    equals the oracle's selection on the same values, bit for bit."""
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp)
    gen = torch.Generator(device="cpu").manual_seed(5)
    for kind in ("ties", "normal"):
        if kind == "ties":
            sc = torch.randint(-4, 5, (w.batch, w.num_kv_heads, g.max_pages), generator=gen)
            sc = sc.float()
            sc[..., ::7] = -0.0  # signed zero must tie with +0
        else:
            sc = torch.randn((w.batch, w.num_kv_heads, g.max_pages), generator=gen) * 50
        scores = sc.cuda()
        for budget, ns, nl in ((w.budget_pages, w.n_sink, w.n_local), (3, 1, 1), (1, 0, 0),
                               (7, 0, 7)):
            sel = torch.empty((w.batch, w.num_kv_heads, budget), device="cuda",
                              dtype=torch.int32)
            cnt = torch.empty((w.batch, w.num_kv_heads), device="cuda", dtype=torch.int32)
            ops.ps_select_topk(g, scores, inp["seq_lens"], budget, ns, nl, sel, cnt)
            torch.cuda.synchronize()
            sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
            for b in range(w.batch):
                n = int(inp["n_pages_host"][b])
                for kv in range(w.num_kv_heads):
                    s64 = sc[b, kv, :n].double().numpy()
                    want, _, _ = ref.select_pages(s64, n, budget, ns, nl)
                    k = min(budget, n)
                    assert int(cnt_h[b, kv]) == k
                    assert list(sel_h[b, kv, :k]) == list(want), (kind, budget, b, kv)
                    assert all(sel_h[b, kv, k:] == -1)


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_decode_on_oracle_selection(cases, w):
    """Sparse decode + merge over the oracle's own page list: partials per
    split and outputs against the oracle (decode parity independent of the
    selection)."""
    _, inp, _, hosts = cases[w.name]
    g = geometry(inp)
    budget = w.budget_pages
    sel = np.full((w.batch, w.num_kv_heads, budget), -1, dtype=np.int32)
    cnt = np.zeros((w.batch, w.num_kv_heads), dtype=np.int32)
    refs = {}
    for (b, kv), hu in hosts.items():
        r = ref.unit_step(hu, 0, 0, budget, w.n_sink, w.n_local)
        sel[b, kv, :len(r["sel"])] = r["sel"]
        cnt[b, kv] = len(r["sel"])
        refs[(b, kv)] = r
    sel_d = torch.from_numpy(sel).cuda()
    cnt_d = torch.from_numpy(cnt).cuda()
    n_splits = min(w.n_splits, budget)
    acc = torch.empty((w.batch, w.num_q_heads, n_splits, w.head_dim), device="cuda")
    ml = torch.empty((w.batch, w.num_q_heads, n_splits, 2), device="cuda")
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), device="cuda")
    ops.ps_sparse_decode(g, inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                         inp["seq_lens"], sel_d, cnt_d, budget, inp["scale"], n_splits, acc, ml)
    ops.ps_combine(g, acc, ml, n_splits, inp["sink"], out, lse)
    torch.cuda.synchronize()
    acc_h, ml_h = acc.cpu().double().numpy(), ml.cpu().double().numpy()
    out_h, lse_h = out.cpu().double().numpy(), lse.cpu().double().numpy()
    grp = w.group
    for (b, kv), hu in hosts.items():
        r = refs[(b, kv)]
        slots = ref.sparse_split_slots(budget, n_splits)
        for i in range(grp):
            h = kv * grp + i
            q_h = hu["q"][0, i].astype(np.float64)
            for s, (lo, hi) in enumerate(slots):
                pages = r["sel"][lo:min(hi, len(r["sel"]))]
                keys = ref.gather_tokens(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                         hu["seq_lens"], 0, 0, pages, 16)
                vals = ref.gather_tokens(hu["v_pool"], hu["kv_dtype"], hu["page_table"],
                                         hu["seq_lens"], 0, 0, pages, 16)
                m, l, a = ref.split_partial(q_h, keys, vals, inp["scale"])
                gm, gl, ga = ml_h[b, h, s, 0], ml_h[b, h, s, 1], acc_h[b, h, s]
                if m == -math.inf:
                    assert gm == -math.inf and gl == 0.0 and not np.any(ga)
                    continue
                assert abs(gm - m) <= 1e-5 * max(1.0, abs(m)), (b, h, s, gm, m)
                assert abs(gl - l) <= 1e-5 * l
                assert rel_l2(ga, a) <= 1e-5
            e = rel_l2(out_h[b, h], r["out"][i])
            assert e <= gate(w), (b, h, e)
            assert abs(lse_h[b, h] - r["lse"][i]) <= 1e-4 * max(1.0, abs(r["lse"][i]))


@pytest.mark.parametrize("w", SMALL, ids=_ids(SMALL))
def test_full_decode_is_exact_attention(cases, w):
    _, inp, _, hosts = cases[w.name]
    g = geometry(inp)
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"])
    out, lse = step.dense(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                          inp["seq_lens"], inp["sink"])
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu().double().numpy(), lse.cpu().double().numpy()
    for (b, kv), hu in hosts.items():
        for i in range(w.group):
            h = kv * w.group + i
            o, l = ref.full_decode(hu, 0, i)
            assert rel_l2(out_h[b, h], o) <= gate(w)
            assert abs(lse_h[b, h] - l) <= 1e-4 * max(1.0, abs(l))


def test_sparse_differs_from_dense(cases):
    """A kernel that ignored the page list would match dense attention; the
    sparse output must not (where the budget is below the page count)."""
    w, inp, res, _ = cases["gqa6_d128_ragged_local"]
    g = geometry(inp)
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"])
    dense, _ = step.dense(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                          inp["seq_lens"], inp["sink"])
    d = dense.cpu().double().numpy()
    assert min(rel_l2(res["out"][b], d[b]) for b in range(w.batch)) > 1e-2


def test_full_budget_sparse_path_equals_dense(cases):
    w, inp, _, _ = cases["tiny_dense"]
    res = run_step(inp)
    g = geometry(inp)
    step = DecodeStep(g, w.budget_pages, 0, 0, w.n_splits, w.dense_splits, inp["scale"])
    assert step.path_for(inp["seq_lens_host"]) == "dense"
    dense, _ = step.dense(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                          inp["seq_lens"], None)
    assert rel_l2(res["out"], dense.cpu().double().numpy()) <= 1e-6


def test_bitwise_deterministic(cases):
    w, inp, res, _ = cases["gqa7_d128_sinkpage_local"]
    res2 = run_step(inp)
    for k in ("sel", "sel_count", "out", "lse", "part_acc", "part_ml"):
        np.testing.assert_array_equal(res[k], res2[k], err_msg=k)
    for b, n in enumerate(inp["n_pages_host"]):  # score slots past n_b are never written
        np.testing.assert_array_equal(res["scores"][b, :, :n], res2["scores"][b, :, :n])


def test_sink_null_equals_minus_inf(cases):
    w, inp, _, _ = cases["gqa8_d64_sink"]
    r_null = run_step(inp, sink=None)
    r_inf = run_step(inp, sink=torch.full((w.num_q_heads,), -math.inf, device="cuda"))
    assert np.array_equal(r_null["out"], r_inf["out"])
    assert np.array_equal(r_null["lse"], r_inf["lse"])


def test_tail_page_refresh_is_incremental(cases):
    """Rebuilding only each request's last page leaves every other metadata
    row untouched and gives the same tail rows as a full build."""
    w, inp, res, hosts = cases["gqa6_d128_ragged_local"]
    g = geometry(inp)
    meta = res["meta"].clone()
    tail = torch.tensor([int(n) - 1 for n in inp["n_pages_host"]], device="cuda",
                        dtype=torch.int32)
    for b in range(w.batch):
        phys = int(inp["page_table"][b, int(inp["n_pages_host"][b]) - 1])
        meta[phys].fill_(7.0)
    ops.ps_build_page_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"], tail, 1, meta)
    torch.cuda.synchronize()
    assert torch.equal(meta, res["meta"])


def test_select_large_candidate_count():
    """More candidates than the select kernel stages in LDS (re-read path)."""
    w = W("long_single", batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64, context=300000,
          budget_pages=64, n_sink=1, n_local=3, needles=4, seed=31, n_splits=8, dense_splits=64)
    inp = wl.make_inputs(w, device="cuda")
    res = run_step(inp)
    hu = unit_host(inp, 0, 0)
    r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
    assert r["n"] > 16384 + 4
    check_selection(res["sel"][0, 0], res["sel_count"][0, 0], r["scores"], r["n"],
                    w.budget_pages, w.n_sink, w.n_local, mag=r["mag"])
    k = int(res["sel_count"][0, 0])
    check_unit_outputs(res, hu, 0, 0, w, w.budget_pages, w.n_sink, w.n_local,
                       sel_dev=res["sel"][0, 0, :k])


@pytest.mark.parametrize("max_pages", [1, 512, 513, 4096, 4097, 32768, 65536])
def test_select_register_tiles(max_pages):
    """Selection on given scores at the edges of the per-lane register tiles
    (512 pages per workgroup per step of the tile), with lengths that leave
    partial wavefront segments, against the oracle's selection."""
    from sparse_long_context_page_amd.ops import Geometry
    gen = torch.Generator(device="cpu").manual_seed(max_pages)
    lengths = sorted({1, max(1, max_pages // 3), max(1, max_pages - 1), max_pages})
    batch = len(lengths)
    g = Geometry(batch, 2, 1, 64, max_pages, 1)
    seq = torch.tensor([n * 16 - 5 if n > 1 else 3 for n in lengths], dtype=torch.int32)
    for kind in ("normal", "ties", "narrow"):
        if kind == "ties":
            sc = torch.randint(-3, 4, (batch, 1, max_pages), generator=gen).float()
        elif kind == "narrow":
            # exact fp32 values 1000 + j * 2^-14: the keys differ only in their
            # low 14 bits, so after one 8-bit pass the bin is small and a
            # second pass decides every bit (with some exact ties)
            j = torch.randint(0, 1 << 14, (batch, 1, max_pages), generator=gen)
            sc = 1000.0 + j.float() * 2.0 ** -14
        else:
            sc = torch.randn((batch, 1, max_pages), generator=gen) * 30 + 100
        for budget, ns, nl in ((128, 1, 4), (64, 0, 0), (2, 1, 1)):
            sel = torch.empty((batch, 1, budget), device="cuda", dtype=torch.int32)
            cnt = torch.empty((batch, 1), device="cuda", dtype=torch.int32)
            ops.ps_select_topk(g, sc.cuda(), seq.cuda(), budget, ns, nl, sel, cnt)
            torch.cuda.synchronize()
            sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
            for b, n in enumerate(lengths):
                want, _, _ = ref.select_pages(sc[b, 0, :n].double().numpy(), n, budget, ns, nl)
                k = min(budget, n)
                assert int(cnt_h[b, 0]) == k
                assert list(sel_h[b, 0, :k]) == list(want), (kind, budget, n)
                assert all(sel_h[b, 0, k:] == -1)
