"""Seeded random geometries: every stage of the path against the fp64
oracle, through the C ABI, on shapes drawn from the supported space (group
size 1..8, head dim 64 or 128, bf16 or fp32 pools, one to four KV heads,
ragged lengths from one token, permuted pools and padded page-table rows,
budgets from one page, sink and local pages, one to eight splits, a learned
sink, and page bounds tightened so that the top-delta threshold binds).

Per case:
- metadata bit-exact, scores within SCORE_REL of fp64 (relative to the
  page magnitude: the terms cancel on tightened pages);
- top-k: the fused launch equals the unfused launches bit for bit; the
  selection equals the oracle's outside the ambiguity band; outputs within
  the rel-L2 gate on the device's page list;
- top-delta at a drawn delta: fused equals unfused bit for bit; the selection
  equals the oracle's rule on the device's own scores; outputs within the gate;
- the dense decode within the gate of exact softmax attention;
- with pool-dtype and with 8-bit metadata, in the physical and the logical
  metadata layout: the refresh of the last pages inside the score launch
  equals the build followed by the score, bit for bit; the 8-bit codes equal
  the oracle's directed rounding; scores on them within SCORE_REL of fp64 and
  the top-k selection identical outside the ambiguity band; the logical
  layout's metadata and scores equal the physical layout's bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle as ref
import workloads as wl
from _gpu_helpers import (SCORE_REL, bits, check_meta_unit, check_selection,
                          check_unit_outputs, gate, geometry, rel_l2, score_rel_err, unit_host,
                          unit_meta)
from sparse_long_context_page_amd import DecodeStep, build_meta, ops

pytestmark = pytest.mark.gpu

N_CASES = 64  # the dtype x group x head-dim grid twice
PAGE = 16


def random_case(i: int):
    """Case i of the sweep: (workload, tighten the page bounds or not, delta).
    Pool dtype, group size and head dim run over the full grid (each of the
    32 combinations once per 32 cases); the rest is drawn."""
    rng = np.random.Generator(np.random.PCG64(9000 + i))
    kv = ("bf16", "f32")[(i // 8) % 2]
    grp = i % 8 + 1
    d = (64, 128)[(i // 16) % 2]
    hkv = int(rng.choice([1, 2, 3, 4]))
    batch = int(rng.integers(1, 9))
    shape = rng.integers(0, 3)
    if shape == 0:  # one fixed length
        lens = dict(context=int(rng.integers(1, 3001)))
        hi = lens["context"]
    elif shape == 1:  # ragged range
        lo = int(rng.integers(1, 800))
        hi = int(rng.integers(lo, 3001))
        lens = dict(ctx_range=(lo, hi))
    else:  # explicit lengths around page boundaries and one long row
        picks = [int(rng.choice([1, 15, 16, 17, 32, 33, 255, 256, 257])) for _ in range(batch)]
        picks[int(rng.integers(0, batch))] = int(rng.integers(1000, 3001))
        lens = dict(lengths=tuple(picks))
        hi = max(picks)
    n_hi = -(-hi // PAGE)
    budget = int(rng.integers(1, 41))
    n_sink = int(rng.integers(0, min(2, budget) + 1))
    n_local = int(rng.integers(0, min(4, budget - n_sink) + 1))
    n_splits = int(rng.integers(1, min(8, budget) + 1))
    w = wl.Workload(
        f"rand{i:02d}_{kv}_d{d}_g{grp}_hkv{hkv}_b{batch}_k{budget}_s{n_sink}l{n_local}"
        f"_sp{n_splits}",
        batch=batch, num_q_heads=grp * hkv, num_kv_heads=hkv, head_dim=d,
        budget_pages=budget, n_sink=n_sink, n_local=n_local,
        needles=int(rng.integers(0, 4)), kv_dtype=kv, sink_logits=bool(rng.random() < 0.4),
        permuted_pool=bool(rng.random() < 0.5), max_pages=n_hi + int(rng.integers(0, 20)),
        seed=9100 + i, n_splits=n_splits, dense_splits=int(rng.integers(1, 17)), **lens)
    tighten = bool(rng.random() < 0.5)
    delta = float(rng.choice([0.0, 0.25, 1.0, 3.0]))
    return w, tighten, delta


CASES = [random_case(i) for i in range(N_CASES)]


def _say(msg):
    print(msg, flush=True)


def _inputs(w, tighten):
    inp = wl.make_inputs(w, device="cuda")
    if tighten:
        wl.tighten_pages(inp, center_std=2.5, seed=w.seed)
    return inp


def _run(inp, g, meta, delta, fused, n_splits):
    w = inp["workload"]
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, n_splits, w.dense_splits,
                      inp["scale"], fused=fused, delta=delta)
    assert step.fused == fused
    step.sel.fill_(-7)
    step.sel_count.fill_(-7)
    step.scores.zero_()  # entries past a request's last page are not written
    out, lse = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                           inp["seq_lens"], inp["sink"])
    acc, ml = step.partials(step.n_splits)
    torch.cuda.synchronize()
    got = dict(sel=step.sel, cnt=step.sel_count, out=out, lse=lse, scores=step.scores)
    if step.n_splits > 1:  # with one split the fused launch writes no partials
        got.update(acc=acc, ml=ml)
    return {k: v.clone() for k, v in got.items()}


def _fused_equals_unfused(inp, g, meta, delta):
    w = inp["workload"]
    a = _run(inp, g, meta, delta, False, w.n_splits)
    b = _run(inp, g, meta, delta, True, w.n_splits)
    for k in a:
        assert torch.equal(a[k], b[k]), (w.name, delta, k)
    return b


def _host(res):
    return {"out": res["out"].cpu().numpy().astype(np.float64),
            "lse": res["lse"].cpu().numpy().astype(np.float64),
            "sel": res["sel"].cpu().numpy(), "cnt": res["cnt"].cpu().numpy(),
            "scores": res["scores"].cpu().numpy().astype(np.float64)}


def _pseudo_max(hu, n, w):
    if w.budget_pages >= n:
        return ref.pseudo_max(hu["q"][0].astype(np.float64),
                              np.zeros((0, hu["q"].shape[-1])), hu["scale"])
    forced = sorted(set(range(min(w.n_sink, n))) | set(range(max(0, n - w.n_local), n)))
    kf = ref.gather_tokens(hu["k_pool"], hu["kv_dtype"], hu["page_table"], hu["seq_lens"], 0, 0,
                           forced, hu["page_size"])
    return ref.pseudo_max(hu["q"][0].astype(np.float64), kf, hu["scale"])


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_random_geometry(case):
    w, tighten, delta = case
    _say(f"case {w.name} tighten={tighten} delta={delta}")
    inp = _inputs(w, tighten)
    g = geometry(inp)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    torch.cuda.synchronize()

    _say("  top-k: fused vs unfused")
    topk = _host(_fused_equals_unfused(inp, g, meta, None))
    _say("  top-delta: fused vs unfused")
    td = _host(_fused_equals_unfused(inp, g, meta, delta))
    _say("  dense decode")
    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"])
    d_out, d_lse = step.dense(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                              inp["seq_lens"], inp["sink"])
    torch.cuda.synchronize()
    d_out, d_lse = d_out.cpu().numpy().astype(np.float64), d_lse.cpu().numpy()

    _say("  oracle")
    scale32 = float(np.float32(inp["scale"]))
    worst_score = worst_k = worst_td = worst_dense = 0.0
    fewer = 0
    for b in range(w.batch):
        n = int(inp["n_pages_host"][b])
        for kv in range(w.num_kv_heads):
            hu = unit_host(inp, b, kv)
            check_meta_unit(inp, meta, hu, b, kv)
            r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
            worst_score = max(worst_score, score_rel_err(topk["scores"][b, kv, :n], r["scores"],
                                                         mag=r["mag"]))

            # top-k end to end
            k = int(topk["cnt"][b, kv])
            check_selection(topk["sel"][b, kv], k, r["scores"], n, w.budget_pages, w.n_sink,
                            w.n_local, mag=r["mag"])
            e, _ = check_unit_outputs(topk, hu, b, kv, w, w.budget_pages, w.n_sink, w.n_local,
                                      sel_dev=topk["sel"][b, kv, :k])
            worst_k = max(worst_k, e)

            # top-delta: the oracle's rule on the device's scores
            mt = _pseudo_max(hu, n, w)
            want, _, _, tau = ref.select_pages_topdelta(td["scores"][b, kv, :n], n,
                                                        w.budget_pages, w.n_sink, w.n_local,
                                                        np.float32(inp["scale"]), mt, delta)
            k = int(td["cnt"][b, kv])
            got = [int(x) for x in td["sel"][b, kv, :k]]
            assert all(int(x) == -1 for x in td["sel"][b, kv, k:])
            assert got == sorted(got) and len(set(got)) == k
            near = set()
            if tau is not None:  # pages within 1e-12 of the threshold may go either way
                near = {p for p in range(n) if abs(scale32 * td["scores"][b, kv, p] - tau)
                        <= 1e-12 * max(abs(tau), 1.0)}
            assert set(got) - near == set(int(x) for x in want) - near, (b, kv)
            fewer += k < min(w.budget_pages, n)
            e, _ = check_unit_outputs(td, hu, b, kv, w, w.budget_pages, w.n_sink, w.n_local,
                                      sel_dev=td["sel"][b, kv, :k])
            worst_td = max(worst_td, e)

            # dense decode: exact attention over every token of the unit's heads
            for i in range(w.group):
                h = kv * w.group + i
                o, l = ref.full_decode(hu, 0, i)
                e = rel_l2(d_out[b, h], o)
                assert e <= gate(w), (b, h, e)
                assert abs(d_lse[b, h] - l) <= 1e-4 * max(1.0, abs(l)), (b, h)
                worst_dense = max(worst_dense, e)

    assert worst_score <= SCORE_REL, worst_score
    _say(f"  score rel {worst_score:.2e}, rel-L2 top-k {worst_k:.2e} top-delta {worst_td:.2e} "
         f"dense {worst_dense:.2e} (gate {gate(w):.0e}); top-delta units below budget: {fewer}")


@pytest.mark.parametrize("meta_layout", ["physical", "logical"])
@pytest.mark.parametrize("meta_format", ["kv", "fp8"])
@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_random_geometry_refresh_and_meta_format(case, meta_format, meta_layout):
    w, tighten, _ = case
    _say(f"case {w.name} tighten={tighten} meta={meta_format} layout={meta_layout}")
    inp = _inputs(w, tighten)
    g = geometry(inp, meta_format, meta_layout)
    full = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    want = torch.empty((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
    ops.ps_score_pages(g, inp["q"], full, inp["page_table"], inp["seq_lens"], want)
    stale = full.clone()
    # the last pages' metadata as if built before the last token was appended
    one = 0x38 if meta_format == "fp8" else 1.0  # 1.0 in E4M3 or in the pool dtype
    for b, n in enumerate(inp["n_pages_host"]):
        if meta_layout == "logical":
            stale[b, :, int(n) - 1] = one
        else:
            stale[int(inp["page_table"][b, int(n) - 1])] = one
    got = torch.full_like(want, float("nan"))
    _say("  refresh score")
    ops.ps_refresh_score_pages(g, inp["q"], inp["k_pool"], stale, inp["page_table"],
                               inp["seq_lens"], got)
    torch.cuda.synchronize()
    assert torch.equal(bits(stale), bits(full))
    for b, n in enumerate(inp["n_pages_host"]):
        assert torch.equal(got[b, :, :int(n)], want[b, :, :int(n)]), b
    if meta_layout == "logical":
        # the same metadata and scores as the physical layout, bit for bit
        gp = geometry(inp, meta_format, "physical")
        phys_meta = build_meta(gp, inp["k_pool"], inp["page_table"], inp["seq_lens"])
        phys_scores = torch.empty_like(want)
        ops.ps_score_pages(gp, inp["q"], phys_meta, inp["page_table"], inp["seq_lens"],
                           phys_scores)
        torch.cuda.synchronize()
        for b, n in enumerate(inp["n_pages_host"]):
            for kv in range(w.num_kv_heads):
                assert torch.equal(bits(unit_meta(inp, full, b, kv)),
                                   bits(unit_meta(inp, phys_meta, b, kv))), (b, kv)
            assert torch.equal(want[b, :, :int(n)], phys_scores[b, :, :int(n)]), b

    step = DecodeStep(g, w.budget_pages, w.n_sink, w.n_local, w.n_splits, w.dense_splits,
                      inp["scale"])
    step.sel.fill_(-7)
    _say("  top-k step")
    step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], full, inp["page_table"],
                inp["seq_lens"], inp["sink"])
    torch.cuda.synchronize()
    sc, sel, cnt = (step.scores.cpu().numpy().astype(np.float64), step.sel.cpu().numpy(),
                    step.sel_count.cpu().numpy())
    meta_h = full.cpu()
    _say("  oracle")
    worst = 0.0
    for b in range(w.batch):
        n = int(inp["n_pages_host"][b])
        for kv in range(w.num_kv_heads):
            hu = unit_host(inp, b, kv, meta_format=meta_format)
            if meta_format == "fp8":
                kmax, kmin = ref.unit_page_meta(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                                hu["seq_lens"], 0, 0, hu["page_size"])
                cmax, cmin = ref.fp8_bounds(kmax, kmin)
                dev = unit_meta(inp, meta_h, b, kv).numpy()
                np.testing.assert_array_equal(dev[:, 0], cmax, err_msg=f"kmax b={b} g={kv}")
                np.testing.assert_array_equal(dev[:, 1], cmin, err_msg=f"kmin b={b} g={kv}")
            else:
                check_meta_unit(inp, full, hu, b, kv)
            r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
            worst = max(worst, score_rel_err(sc[b, kv, :n], r["scores"], mag=r["mag"]))
            check_selection(sel[b, kv], cnt[b, kv], r["scores"], n, w.budget_pages, w.n_sink,
                            w.n_local, mag=r["mag"])
    _say(f"  score rel {worst:.2e}")
    assert worst <= SCORE_REL, worst
