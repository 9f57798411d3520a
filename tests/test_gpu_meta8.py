"""8-bit metadata (E4M3 bounds: kmax rounded up, kmin rounded down) through
the C ABI against the fp64 oracle, on bf16 pools (matrix-core score) and fp32
pools (vector-ALU score): every code decodes to its value, the codes
equal the oracle's directed rounding bit for bit, scores match the fp64 bound
on the 8-bit values, selections are identical outside the ambiguity band,
outputs are within the rel-L2 gate, and the refresh inside the score launch
equals the metadata build followed by the score, bit for bit."""

import numpy as np
import pytest
import torch

import oracle as ref
import workloads as wl
from _gpu_helpers import (SCORE_REL, check_selection, check_unit_outputs, gate, geometry,
                          run_step, score_rel_err, unit_host)
from sparse_long_context_page_amd import Geometry, build_meta, ops
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

CASES = SMALL


@pytest.mark.parametrize("kv", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_every_code_decodes_to_its_value(d, kv):
    """A request per coordinate, its query one-hot on that coordinate, all
    reading the same pages whose kmax rows hold every finite code and whose
    kmin is -448: score[b, p] = value of the code at (p, d=b). This pins the
    widening and the coordinate assignment of the score kernel together."""
    t = ref.fp8_e4m3_table()
    codes = np.array([c if not np.isnan(t[c]) else 0 for c in range(256)], dtype=np.uint8)
    n_pages = 256 // d
    meta = np.zeros((n_pages, 1, 2, d), dtype=np.uint8)
    meta[:, 0, 0, :] = codes.reshape(n_pages, d)
    meta[:, 0, 1, :] = 0xFE  # -448
    g = Geometry(d, 1, 1, d, n_pages, n_pages, kv, 16, "fp8")
    q = torch.eye(d, dtype=torch.float32).reshape(d, 1, d).cuda()
    table = torch.arange(n_pages, dtype=torch.int32).repeat(d, 1).cuda()
    lens = torch.full((d,), 16 * n_pages, dtype=torch.int32).cuda()
    scores = torch.full((d, 1, n_pages), float("nan")).cuda()
    ops.ps_score_pages(g, q, torch.from_numpy(meta).cuda(), table, lens, scores)
    torch.cuda.synchronize()
    got = scores[:, 0, :].cpu().numpy().T  # [page, d]
    want = t[codes].reshape(n_pages, d)
    np.testing.assert_array_equal(got, want)


@pytest.fixture(scope="module")
def cases():
    out = {}
    for w in CASES:
        inp = wl.make_inputs(w, device="cuda")
        res = run_step(inp, meta_format="fp8")
        units = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
        out[w.name] = (w, inp, res, {u: unit_host(inp, *u, meta_format="fp8") for u in units})
    return out


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_codes_bit_exact(cases, w):
    _, inp, res, hosts = cases[w.name]
    for (b, g), hu in hosts.items():
        n = int(inp["n_pages_host"][b])
        phys = inp["page_table"][b, :n].long()
        dev = res["meta"][phys, g].cpu().numpy()  # [n, 2, D] uint8
        kmax, kmin = ref.unit_page_meta(hu["k_pool"], hu["kv_dtype"], hu["page_table"],
                                        hu["seq_lens"], 0, 0, hu["page_size"])
        cmax, cmin = ref.fp8_bounds(kmax, kmin)
        np.testing.assert_array_equal(dev[:, 0], cmax, err_msg=f"kmax codes b={b} g={g}")
        np.testing.assert_array_equal(dev[:, 1], cmin, err_msg=f"kmin codes b={b} g={g}")


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_scores_match_fp64(cases, w):
    _, inp, res, hosts = cases[w.name]
    worst = 0.0
    for (b, g), hu in hosts.items():
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
        worst = max(worst, score_rel_err(res["scores"][b, g, :r["n"]].astype(np.float64),
                                         r["scores"], mag=r["mag"]))
    print(f"{w.name}: max score rel err {worst:.3e}")
    assert worst <= SCORE_REL


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_selection_and_outputs(cases, w):
    _, inp, res, hosts = cases[w.name]
    worst = 0.0
    for (b, g), hu in hosts.items():
        r = ref.unit_step(hu, 0, 0, w.budget_pages, w.n_sink, w.n_local)
        check_selection(res["sel"][b, g], res["sel_count"][b, g], r["scores"], r["n"],
                        w.budget_pages, w.n_sink, w.n_local, mag=r["mag"])
        k = int(res["sel_count"][b, g])
        e, _ = check_unit_outputs(res, hu, b, g, w, w.budget_pages, w.n_sink, w.n_local,
                                  sel_dev=res["sel"][b, g, :k])
        worst = max(worst, e)
    print(f"{w.name}: max rel-L2 {worst:.3e} (gate {gate(w)})")


@pytest.mark.parametrize("w", CASES + [wl.B32_64K], ids=[w.name for w in CASES + [wl.B32_64K]])
def test_refresh_score_equals_meta_then_score_bitwise(w):
    inp = wl.make_inputs(w, device="cuda")
    g = geometry(inp, "fp8")
    full = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
    assert full.dtype == torch.uint8
    want = torch.empty((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
    ops.ps_score_pages(g, inp["q"], full, inp["page_table"], inp["seq_lens"], want)
    stale = full.clone()
    tails = [int(inp["page_table"][b, int(n) - 1]) for b, n in enumerate(inp["n_pages_host"])]
    stale[tails] = 0x38  # 1.0: what the pages held before the last token was appended
    got = torch.full_like(want, float("nan"))
    ops.ps_refresh_score_pages(g, inp["q"], inp["k_pool"], stale, inp["page_table"],
                               inp["seq_lens"], got)
    torch.cuda.synchronize()
    assert torch.equal(stale, full)
    for b, n in enumerate(inp["n_pages_host"]):
        assert torch.equal(got[b, :, :int(n)], want[b, :, :int(n)]), (w.name, b)


@pytest.mark.parametrize("w", [wl.B8_16K, wl.TINY], ids=["b8_bf16", "tiny_f32"])
def test_fp8_scores_bound_the_kv_dtype_scores(w):
    """On the same inputs the score on 8-bit metadata is >= the score on
    metadata in the pool's dtype for every page (the 8-bit box contains the
    exact one), and both are finite."""
    inp = wl.make_inputs(w, device="cuda")
    s = {}
    for fmt in ("kv", "fp8"):
        g = geometry(inp, fmt)
        meta = build_meta(g, inp["k_pool"], inp["page_table"], inp["seq_lens"])
        sc = torch.empty((g.batch, g.num_kv_heads, g.max_pages), device="cuda")
        ops.ps_score_pages(g, inp["q"], meta, inp["page_table"], inp["seq_lens"], sc)
        s[fmt] = sc
    torch.cuda.synchronize()
    for b, n in enumerate(inp["n_pages_host"]):
        a, c = s["kv"][b, :, :int(n)], s["fp8"][b, :, :int(n)]
        assert torch.isfinite(c).all()
        # the device sums in fp32: allow its rounding on top of the exact ordering
        assert (c >= a - 1e-6 * a.abs()).all()
