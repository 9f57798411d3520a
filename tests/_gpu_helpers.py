"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle as ref
import workloads as wl
from sparse_long_context_page_amd import DecodeStep, Geometry, build_meta, ops

BF16_GATE = 2e-3  # rel-L2 per (request, query head), bf16 K/V, fp32 accumulation
F32_GATE = 1e-5   # same, fp32 K/V
# device fp32 score vs fp64, relative to the page's magnitude (the oracle's
# score_magnitudes: the sum of the terms' absolute values, the scale of any
# fp32 summation's error; equal to |score| when the terms do not cancel);
# well inside the 1e-6 ambiguity band
SCORE_REL = 5e-7


def gate(w) -> float:
    return BF16_GATE if w.kv_dtype == "bf16" else F32_GATE


def geometry(inp, meta_format="kv", meta_layout="physical") -> Geometry:
    return Geometry.of(inp["q"], inp["k_pool"], inp["page_table"], meta_format, meta_layout)


def unit_meta(inp, meta, b, g):
    """The metadata of the n_b pages of (request b, KV head g), [n_b, 2, D],
    from either layout: [P_phys, Hkv, 2, D] (gathered through the page
    table) or [B, Hkv, max_pages, 2, D] (the request's own slots)."""
    n = int(inp["n_pages_host"][b])
    if meta.dim() == 5:
        return meta[b, g, :n]
    return meta[inp["page_table"][b, :n].long().to(meta.device), g]


def bits(t):
    """Integer view of a tensor, so that equality is bit equality (NaN
    patterns in never-written slots included)."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def unit_host(inp, b, g, meta_format="kv"):
    """Oracle view of one (request, KV head): the unit's pages gathered into a
    compact host pool with an identity page table (plain torch indexing).
    meta_format "fp8": the oracle scores the 8-bit bounds."""
    w = inp["workload"]
    grp = w.group
    n = int(inp["n_pages_host"][b])
    phys = inp["page_table"][b, :n].long()
    k = inp["k_pool"][phys, g:g + 1]
    v = inp["v_pool"][phys, g:g + 1]
    sink = None if inp["sink"] is None else inp["sink"][g * grp:(g + 1) * grp].cpu().numpy()
    return {
        "q": inp["q"][b:b + 1, g * grp:(g + 1) * grp].cpu().numpy(),
        "k_pool": wl.kv_bits_numpy(k),
        "v_pool": wl.kv_bits_numpy(v),
        "kv_dtype": w.kv_dtype,
        "page_table": np.arange(n, dtype=np.int32)[None, :],
        "seq_lens": inp["seq_lens"][b:b + 1].cpu().numpy(),
        "page_size": w.page_size,
        "scale": inp["scale"],
        "sink": sink,
        "meta_format": ref.FP8_E4M3 if meta_format == "fp8" else None,
    }


def run_step(inp, budget=None, n_splits=None, n_sink=None, n_local=None, sink="input",
             meta_format="kv", meta_layout="physical"):
    """Metadata build + sparse step on the device; returns host copies."""
    w = inp["workload"]
    g = geometry(inp, meta_format, meta_layout)
    budget = w.budget_pages if budget is None else budget
    step = DecodeStep(g, budget, w.n_sink if n_sink is None else n_sink,
                      w.n_local if n_local is None else n_local,
                      n_splits=w.n_splits if n_splits is None else n_splits,
                      dense_splits=w.dense_splits, scale=inp["scale"])
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    s = inp["sink"] if sink == "input" else sink
    out, lse = step.sparse(inp["q"], inp["k_pool"], inp["v_pool"], meta, inp["page_table"],
                           inp["seq_lens"], s)
    acc, ml = step.partials(step.n_splits)
    torch.cuda.synchronize()
    return {
        "step": step,
        "meta": meta,
        "scores": step.scores.cpu().numpy(),
        "sel": step.sel.cpu().numpy(),
        "sel_count": step.sel_count.cpu().numpy(),
        "out": out.cpu().numpy().astype(np.float64),
        "lse": lse.cpu().numpy().astype(np.float64),
        "part_acc": acc.cpu().numpy().astype(np.float64),
        "part_ml": ml.cpu().numpy().astype(np.float64),
    }


def check_meta_unit(inp, meta, hu, b, g):
    """Device metadata of one unit equals the oracle's, value for value."""
    dev = wl.kv_bits_numpy(unit_meta(inp, meta, b, g))  # [n, 2, D]
    kmax, kmin = ref.unit_page_meta(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                    hu["seq_lens"], 0, 0, hu["page_size"])
    got_max = ref.widen(np.ascontiguousarray(dev[:, 0]), hu["kv_dtype"])
    got_min = ref.widen(np.ascontiguousarray(dev[:, 1]), hu["kv_dtype"])
    assert np.array_equal(got_max, kmax), f"kmax mismatch b={b} g={g}"
    assert np.array_equal(got_min, kmin), f"kmin mismatch b={b} g={g}"


def score_rel_err(dev_scores, ref_scores, mag=None):
    """Largest |device - fp64| over the pages, relative to the page's
    magnitude when given (else to |fp64|)."""
    dev = np.asarray(dev_scores, dtype=np.float64)
    den = np.abs(ref_scores) if mag is None else np.maximum(np.abs(ref_scores), mag)
    if dev.size == 0:
        return 0.0
    return float(np.max(np.abs(dev - ref_scores) / np.maximum(den, 1e-30)))


def check_selection(sel_row, count, scores_ref, n, budget, n_sink, n_local, mag=None):
    """Device page list vs the oracle: same count, ascending, -1 padded,
    forced pages present, identical outside the ambiguity band.
    Returns (ambiguous count, whether the lists differ inside the band)."""
    k = min(budget, n)
    assert int(count) == k, (count, k)
    row = [int(x) for x in sel_row[:k]]
    assert all(int(x) == -1 for x in sel_row[k:])
    assert row == sorted(row) and len(set(row)) == k
    assert all(0 <= p < n for p in row)
    sel_o, forced, _ = ref.select_pages(scores_ref, n, budget, n_sink, n_local)
    amb, _ = ref.ambiguous_pages(scores_ref, n, budget, n_sink, n_local, mag=mag)
    assert set(forced) <= set(row)
    assert set(row) - amb == set(int(p) for p in sel_o) - amb, "selection differs outside band"
    return len(amb), set(row) != set(int(p) for p in sel_o)


def rel_l2(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def check_unit_outputs(res, hu, b, g, w, budget, n_sink, n_local, sel_dev=None):
    """Oracle step for one unit (on the device's page list when given) vs the
    device output rows of the unit's query heads. Returns max rel-L2."""
    r = ref.unit_step(hu, 0, 0, budget, n_sink, n_local, sel_override=sel_dev)
    grp = w.group
    worst = 0.0
    for i in range(grp):
        h = g * grp + i
        e = rel_l2(res["out"][b, h], r["out"][i])
        worst = max(worst, e)
        assert e <= gate(w), f"rel-L2 {e} > {gate(w)} at b={b} h={h}"
        assert abs(res["lse"][b, h] - r["lse"][i]) <= 1e-4 * max(1.0, abs(r["lse"][i]))
    return worst, r
