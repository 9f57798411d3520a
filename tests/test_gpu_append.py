"""Incremental metadata on append (ps_build_page_meta with page_begin) against
the oracle's pool-wide build.

Tokens are appended to every request (1, 16 or 17 of them: inside the last
page, exactly one page, across a page boundary), the new pages mapped to
fresh physical pages; the device then rebuilds only the pages the new tokens
touch (page_begin[b] = the old last page). The device metadata of the new
state must equal, bit for bit, the oracle's page_meta_pool of the new state
on every mapped page (pool-dtype bounds exact; 8-bit bounds as the oracle's
directed rounding of them), the oracle's incremental build (pages_of = the
touched pages) on the touched ones, and the rows no request maps, or that no
new token touches, must be unchanged. In the logical metadata layout the
same holds slot by slot: the slot (b, g, p) holds the entry of the page
page_table[b, p]. ("Don't read the haystack", section "Part two: the
skipping": the page summaries are maintained as tokens append.)
"""

import numpy as np
import pytest
import torch

import oracle as ref
import workloads as wl
from _gpu_helpers import geometry
from _pins import _append_tokens
from sparse_long_context_page_amd import build_meta, ops

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16", 128, "kv", "physical"), ("bf16", 64, "kv", "physical"),
    ("f32", 128, "kv", "physical"), ("f32", 64, "kv", "physical"),
    ("bf16", 128, "fp8", "physical"), ("f32", 64, "fp8", "physical"),
    ("bf16", 128, "kv", "logical"), ("f32", 64, "kv", "logical"),
    ("bf16", 64, "fp8", "logical"), ("f32", 128, "fp8", "logical"),
]


def _device_pool(bits: np.ndarray, kv_dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if kv_dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


@pytest.mark.parametrize("kv,d,meta_format,layout", CASES,
                         ids=[f"{a}-d{b}-{c}-{e}" for a, b, c, e in CASES])
def test_incremental_build_equals_oracle_pool(kv, d, meta_format, layout):
    print(f"\n[append] kv={kv} d={d} meta={meta_format} layout={layout}", flush=True)
    logical = layout == "logical"
    w = wl.Workload("append", batch=6, num_q_heads=8, num_kv_heads=2, head_dim=d,
                    ctx_range=(1, 600), budget_pages=4, kv_dtype=kv, permuted_pool=True,
                    max_pages=48, seed=4242)
    inp = wl.make_inputs(w, device="cuda")
    h = wl.host_inputs(inp)
    g = geometry(inp, meta_format, layout)
    meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    torch.cuda.synchronize()

    extra = [(1, 16, 17)[b % 3] for b in range(w.batch)]
    h2 = _append_tokens(h, extra)
    p_old, p_new = h["k_pool"].shape[0], h2["k_pool"].shape[0]
    k2 = _device_pool(h2["k_pool"], kv)
    table2 = torch.from_numpy(h2["page_table"]).cuda()
    lens2 = torch.from_numpy(h2["seq_lens"]).cuda()
    g2 = ops.Geometry(w.batch, w.num_q_heads, w.num_kv_heads, d, table2.shape[1], p_new,
                      k2.dtype, w.page_size, meta_format, layout)
    meta2 = torch.empty(ops.meta_shape(g2), device="cuda", dtype=g2.meta_dtype)
    if meta_format == "fp8":
        meta2.fill_(0x7F)  # a NaN code: every fresh row the build misses stays visible
    else:
        meta2.fill_(float("nan"))
    if logical:
        meta2[:, :, :g.max_pages].copy_(meta)
    else:
        meta2[:p_old].copy_(meta)
    before = meta2.clone()

    n_old = [ref.num_pages(int(x), w.page_size) for x in h["seq_lens"]]
    n_new = [ref.num_pages(int(x), w.page_size) for x in h2["seq_lens"]]
    begin = torch.tensor([n - 1 for n in n_old], dtype=torch.int32, device="cuda")
    n_pages = max(b_ - a_ + 1 for a_, b_ in zip(n_old, n_new))
    ops.ps_build_page_meta(g2, k2, table2, lens2, begin, n_pages, meta2)
    torch.cuda.synchronize()

    full = ref.page_meta_pool(h2["k_pool"], kv, h2["page_table"], h2["seq_lens"], w.page_size)
    touched = {b: list(range(n_old[b] - 1, n_new[b])) for b in range(w.batch)}
    inc = ref.page_meta_pool(h2["k_pool"], kv, h2["page_table"], h2["seq_lens"], w.page_size,
                             pages_of=touched)
    dev = meta2.cpu()
    dev_np = dev.numpy() if meta_format == "fp8" else wl.kv_bits_numpy(dev)

    def expect(kmax, kmin):
        if meta_format == "fp8":
            return ref.fp8_bounds(kmax, kmin)
        return kmax, kmin

    def rows(x):
        if meta_format == "fp8":
            return x[0], x[1]
        return (ref.widen(np.ascontiguousarray(x[0]), kv),
                ref.widen(np.ascontiguousarray(x[1]), kv))

    # where the entry of (physical page, head) sits: one place per physical
    # page, or every logical slot that maps the page
    if logical:
        slots = {}
        for b in range(w.batch):
            for p in range(n_new[b]):
                for g_ in range(w.num_kv_heads):
                    slots.setdefault((int(h2["page_table"][b, p]), g_), []).append((b, g_, p))
    else:
        slots = {key: [key] for key in full}

    for (phys, g_), (kmax, kmin) in full.items():
        ex, en = expect(kmax, kmin)
        for at in slots[(phys, g_)]:
            gx, gn = rows(dev_np[at])
            assert np.array_equal(gx, ex) and np.array_equal(gn, en), f"page {phys} at {at}"
    for (phys, g_), (kmax, kmin) in inc.items():
        ex, en = expect(kmax, kmin)
        for at in slots[(phys, g_)]:
            gx, gn = rows(dev_np[at])
            assert np.array_equal(gx, ex) and np.array_equal(gn, en), f"touched {phys} at {at}"
    # every other row or slot is unchanged
    changed = torch.zeros(dev.shape[:-2], dtype=torch.bool)
    if logical:
        for b in range(w.batch):
            changed[b, :, n_old[b] - 1:n_new[b]] = True
    else:
        changed[sorted({phys for phys, _ in inc})] = True
    keep = ~changed
    assert torch.equal(dev[keep].view(torch.uint8), before.cpu()[keep].view(torch.uint8))
    print(f"[append] {len(full)} mapped entries equal, {len(inc)} rebuilt", flush=True)
