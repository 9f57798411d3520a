"""HIP path vs the fp64 oracle at the full sizes of the four bf16 workloads,
in the launch configuration the benchmark times (the workload's split counts):

  b8_16k_needles_sink_page        8 x 16k tokens, GQA 6, sink page kept
  b32_64k_needles_local4          32 x 64k tokens, GQA 6, last 4 pages kept
  b16_32k_learned_sink            16 x 32k tokens, GQA 8, d64, learned sink logits
  b64_ragged_4k_128k_shared_pool  64 requests of 4k..128k tokens, GQA 7,
                                  permuted shared pool, partial last pages

The oracle computes sampled (request, KV head) units one by one: metadata bit
for bit, scores against fp64, the page list identical outside the ambiguity
band, and the outputs within the rel-L2 gate. Properties that hold at any size
(count, order, padding, forced pages) are checked on every unit.
"""

import numpy as np
import pytest
import torch

import oracle as ref
import workloads as wl
from _gpu_helpers import (SCORE_REL, check_meta_unit, check_selection, check_unit_outputs,
                          gate, geometry, rel_l2, run_step, score_rel_err, unit_host)
from sparse_long_context_page_amd import DecodeStep

pytestmark = pytest.mark.gpu

FULL = [wl.B8_16K, wl.B32_64K, wl.SINK, wl.RAGGED]


def _sample_units(w, k=3):
    rng = np.random.default_rng(w.seed + 77)
    units = {(0, 0), (w.batch - 1, w.num_kv_heads - 1)}
    while len(units) < k:
        units.add((int(rng.integers(w.batch)), int(rng.integers(w.num_kv_heads))))
    return sorted(units)


@pytest.fixture(scope="module", params=FULL, ids=[w.name for w in FULL])
def full(request):
    w = request.param
    print(f"\n[full-size] generating {w.name}", flush=True)
    inp = wl.make_inputs(w, device="cuda")
    res = run_step(inp)
    yield w, inp, res
    del inp, res
    torch.cuda.empty_cache()


def test_every_unit_page_list_is_well_formed(full):
    w, inp, res = full
    for b in range(w.batch):
        n = int(inp["n_pages_host"][b])
        k = min(w.budget_pages, n)
        forced = set(range(min(w.n_sink, n))) | set(range(max(0, n - w.n_local), n))
        for g in range(w.num_kv_heads):
            row = res["sel"][b, g]
            assert int(res["sel_count"][b, g]) == k
            kept = [int(x) for x in row[:k]]
            assert kept == sorted(set(kept)) and 0 <= kept[0] and kept[-1] < n
            assert all(int(x) == -1 for x in row[k:])
            if k < n:
                assert forced <= set(kept)


def test_sampled_units_match_oracle(full):
    w, inp, res = full
    worst, n_amb = 0.0, 0
    for b, g in _sample_units(w):
        print(f"[full-size] {w.name} unit b={b} g={g}", flush=True)
        hu = unit_host(inp, b, g)
        check_meta_unit(inp, res["meta"], hu, b, g)
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
        n = r["n"]
        assert score_rel_err(res["scores"][b, g, :n], r["scores"], mag=r["mag"]) <= SCORE_REL
        amb, differs = check_selection(res["sel"][b, g], res["sel_count"][b, g], r["scores"], n,
                                       w.budget_pages, w.n_sink, w.n_local, mag=r["mag"])
        n_amb += amb
        k = int(res["sel_count"][b, g])
        e, _ = check_unit_outputs(res, hu, b, g, w, w.budget_pages, w.n_sink, w.n_local,
                                  sel_dev=res["sel"][b, g, :k] if differs else None)
        worst = max(worst, e)
    print(f"[full-size] {w.name}: max rel-L2 {worst:.3e}, ambiguous pages {n_amb}")


def test_dense_decode_matches_exact_attention(full):
    w, inp, _ = full
    if w.name not in (wl.B8_16K.name, wl.B32_64K.name):
        pytest.skip("the dense check runs on the two uniform-length GQA-6 workloads")
    step = DecodeStep(geometry(inp), w.budget_pages, w.n_sink, w.n_local, w.n_splits,
                      w.dense_splits, inp["scale"])
    out, lse = step.dense(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                          inp["seq_lens"], inp["sink"])
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu().double().numpy(), lse.cpu().double().numpy()
    for b, g in _sample_units(w, k=2):
        hu = unit_host(inp, b, g)
        for i in range(w.group):
            h = g * w.group + i
            o, l = ref.full_decode(hu, 0, i)
            assert rel_l2(out_h[b, h], o) <= gate(w)
            assert abs(lse_h[b, h] - l) <= 1e-4 * max(1.0, abs(l))


def test_sampled_units_match_oracle_with_8bit_metadata(full):
    """The same step with 8-bit metadata bounds, at full size: the codes of
    the sampled units bit for bit against the oracle's directed rounding,
    scores against fp64 on the 8-bit values, page lists and outputs."""
    w, inp, _ = full
    res = run_step(inp, meta_format="fp8")
    for b, g in _sample_units(w, k=2):
        print(f"[full-size fp8] {w.name} unit b={b} g={g}", flush=True)
        hu = unit_host(inp, b, g, meta_format="fp8")
        n = int(inp["n_pages_host"][b])
        phys = inp["page_table"][b, :n].long()
        dev = res["meta"][phys, g].cpu().numpy()
        kmax, kmin = ref.unit_page_meta(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                        hu["seq_lens"], 0, 0, hu["page_size"])
        cmax, cmin = ref.fp8_bounds(kmax, kmin)
        assert np.array_equal(dev[:, 0], cmax) and np.array_equal(dev[:, 1], cmin)
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
        assert score_rel_err(res["scores"][b, g, :n], r["scores"], mag=r["mag"]) <= SCORE_REL
        _, differs = check_selection(res["sel"][b, g], res["sel_count"][b, g], r["scores"], n,
                                     w.budget_pages, w.n_sink, w.n_local, mag=r["mag"])
        k = int(res["sel_count"][b, g])
        check_unit_outputs(res, hu, b, g, w, w.budget_pages, w.n_sink, w.n_local,
                           sel_dev=res["sel"][b, g, :k] if differs else None)
    del res
    torch.cuda.empty_cache()
