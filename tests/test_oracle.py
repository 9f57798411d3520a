"""The fp64 oracle pinned to facts it does not compute itself (CPU only).

Pins: admissibility of the bound, tight and closed-form cases of the bound,
selection re-derived by rank counting and by exhaustive search, exact
attention through torch's SDPA in fp64 (dense case, restricted-mask case and
sink as an extra zero key), the sink's closed form, split/merge invariance and
invariance to the physical page layout. The mutation tests at the end plant a
plausible mistake in the oracle and check that one of these pins catches it.
"""

import math

import numpy as np
import pytest

import oracle as ref
import workloads as wl
from _pins import (check_dense_is_exact_attention, check_fp8_bound_admissible, check_fp8_decode,
                   check_topdelta, check_topdelta_no_forced_is_topk, tight_small_inputs,
                   check_fp8_directed_rounding, check_meta_bounds, check_meta_pool, check_restricted_reference,
                   check_score_admissible, check_score_closed_forms, check_selection_bruteforce,
                   check_selection_rank_count, check_sink, check_split_invariance,
                   check_split_ranges, small_inputs)


@pytest.fixture(scope="module")
def small():
    return small_inputs()


@pytest.fixture(scope="module")
def tiny():
    inp = wl.make_inputs(wl.TINY, device="cpu")
    return inp, wl.host_inputs(inp)


def test_widen_bf16_exact():
    import torch
    x = torch.tensor([1.0, -2.5, 3.140625, 1e-20, -7.0e4], dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ref.widen(bits, ref.BF16), x.float().numpy().astype(np.float64))
    with pytest.raises(TypeError):
        ref.widen(np.zeros(3, np.float32), ref.BF16)


def test_page_counts():
    assert ref.num_pages(1, 16) == 1
    assert ref.num_pages(16, 16) == 1
    assert ref.num_pages(17, 16) == 2
    assert ref.num_pages(65536, 16) == 4096
    assert ref.page_token_count(17, 1, 16) == 1
    assert ref.page_token_count(32, 1, 16) == 16
    assert ref.page_token_count(40, 3, 16) == 0


def test_meta_bounds(small):
    _, _, h = small
    check_meta_bounds(ref, h)


def test_meta_pool_and_incremental_update(small, tiny):
    check_meta_pool(ref.pagesparse_ref, small[2])
    check_meta_pool(ref.pagesparse_ref, tiny[1])


def test_meta_bounds_fp32(tiny):
    check_meta_bounds(ref, tiny[1])


def test_score_admissible(small):
    _, _, h = small
    assert check_score_admissible(ref, h) >= 0.0


def test_score_admissible_tiny(tiny):
    assert check_score_admissible(ref, tiny[1]) >= 0.0


def test_score_closed_forms():
    check_score_closed_forms(ref)


@pytest.mark.parametrize("group", [1, 2])
def test_topdelta_selection(group):
    w, _, h = tight_small_inputs(group)
    binds = check_topdelta(ref, h, w)
    assert binds > 0  # some cases exercise the cap


@pytest.mark.parametrize("group", [1, 2])
def test_topdelta_threshold_separates_tight_pages(group):
    """On tight pages the threshold keeps fewer pages than the budget for
    some units (the criterion is exercised, not only the cap)."""
    w, _, h = tight_small_inputs(group)
    fewer = 0
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            r = ref.unit_step(h, b, g, w.budget_pages, w.n_sink, w.n_local, delta=0.3)
            fewer += len(r["sel"]) < min(w.budget_pages, r["n"])
    assert fewer > 0


def test_topdelta_no_forced_is_topk():
    w, _, h = tight_small_inputs()
    check_topdelta_no_forced_is_topk(ref, h, w)


def test_fp8_decode():
    check_fp8_decode(ref)


def test_fp8_directed_rounding():
    check_fp8_directed_rounding(ref)


def test_fp8_bound_admissible(small):
    check_fp8_bound_admissible(ref, small[2])


def test_fp8_unit_step_scores_the_8bit_bounds(small):
    """With meta_format = FP8_E4M3 the step ranks pages by the bound on the
    8-bit metadata; attention is unchanged for the same page list."""
    w, _, h = small
    h8 = dict(h, meta_format=ref.FP8_E4M3)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            r16 = ref.unit_step(h, b, g, w.budget_pages, w.n_sink, w.n_local)
            r8 = ref.unit_step(h8, b, g, w.budget_pages, w.n_sink, w.n_local)
            assert np.all(r8["u"] >= r16["u"])
            r16b = ref.unit_step(h, b, g, w.budget_pages, w.n_sink, w.n_local,
                                 sel_override=r8["sel"])
            np.testing.assert_array_equal(r16b["out"], r8["out"])


def test_score_single_token_page_is_tight():
    # a request whose last page holds exactly one valid token: the bound of
    # that page equals q.k of that token for each head
    w, inp, h = small_inputs(ctx_range=(33, 33), batch=1, needles=0)
    kmax, kmin = ref.unit_page_meta(h["k_pool"], h["kv_dtype"], h["page_table"], h["seq_lens"],
                                    0, 1, 16)
    q = h["q"][0, 3:6].astype(np.float64)
    u, _ = ref.unit_scores(q, kmax, kmin)
    key = ref.gather_tokens(h["k_pool"], h["kv_dtype"], h["page_table"], h["seq_lens"], 0, 1,
                            [2], 16)
    assert key.shape[0] == 1
    np.testing.assert_allclose(u[:, 2], q @ key[0], rtol=1e-13)


def test_selection_rank_count(small):
    w, inp, h = small
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            res = ref.unit_step(h, b, g, w.budget_pages, w.n_sink, w.n_local)
            check_selection_rank_count(ref, res["scores"], res["n"], w.budget_pages, w.n_sink,
                                       w.n_local)
            for budget, ns, nl in ((1, 0, 0), (3, 1, 2), (5, 2, 0), (100, 1, 1)):
                check_selection_rank_count(ref, res["scores"], res["n"], budget, ns, nl)


def test_selection_bruteforce():
    check_selection_bruteforce(ref)


def test_selection_ties_to_lower_index():
    s = np.array([1.0, 5.0, 5.0, 5.0, 2.0, 5.0])
    sel, forced, taken = ref.select_pages(s, 6, 3, 0, 0)
    assert list(sel) == [1, 2, 3] and taken == [1, 2, 3]
    sel, _, _ = ref.select_pages(s, 6, 3, 0, 1)  # page 5 forced
    assert list(sel) == [1, 2, 5]


def test_ambiguity_band():
    s = np.array([10.0, 9.0, 8.0 * (1 + 5e-7), 8.0, 1.0])
    amb, s_k = ref.ambiguous_pages(s, 5, 3, 0, 0)
    assert s_k == s[2] and amb == {2, 3}
    amb, _ = ref.ambiguous_pages(s, 5, 2, 0, 0)
    assert amb == {1}


def test_score_magnitudes_hand_example():
    """Two heads, two coordinates, one page: kmax = (2, 3), kmin = (1, 2).
    Head 0, q = (1, -1): terms max(1, 2) = 2 and max(-2, -3) = -2, so the
    bound is 0 and the magnitude 4. Head 1, q = (0.5, 0.5): terms 1 and 1.5,
    bound 2.5, magnitude 2.5. The group takes the larger of each: score 2.5,
    magnitude 4 (from the head whose terms cancel)."""
    q = np.array([[1.0, -1.0], [0.5, 0.5]])
    kmax = np.array([[2.0, 3.0]])
    kmin = np.array([[1.0, 2.0]])
    u, s = ref.unit_scores(q, kmax, kmin)
    assert u.tolist() == [[0.0], [2.5]] and s.tolist() == [2.5]
    assert ref.score_magnitudes(q, kmax, kmin).tolist() == [4.0]


def test_score_magnitudes_without_cancellation_equal_the_score():
    """With q >= 0 and kmin >= 0 every term is non-negative, so the magnitude
    is the score itself; in general it is at least |score| (triangle
    inequality) for every page."""
    rng = np.random.default_rng(3)
    q = np.abs(rng.standard_normal((3, 64)))
    lo = np.abs(rng.standard_normal((20, 64)))
    hi = lo + np.abs(rng.standard_normal((20, 64)))
    _, s = ref.unit_scores(q, hi, lo)
    np.testing.assert_allclose(ref.score_magnitudes(q, hi, lo), s, rtol=1e-15)
    q = rng.standard_normal((4, 128))
    lo = rng.standard_normal((50, 128))
    hi = lo + np.abs(rng.standard_normal((50, 128)))
    _, s = ref.unit_scores(q, hi, lo)
    assert np.all(ref.score_magnitudes(q, hi, lo) >= np.abs(s) * (1 - 1e-15))


def test_fp32_score_error_is_bounded_by_the_magnitude():
    """A left-to-right fp32 sum of the D exact terms stays within
    D * 2^-24 * magnitude of the fp64 score (the forward error bound of
    recursive summation) on pages whose terms cancel almost completely, while
    its error relative to the score itself is far larger there."""
    rng = np.random.default_rng(4)
    d = 128
    centre = rng.standard_normal((200, d)) * 2.5
    lo = (centre - 0.05).astype(np.float32).astype(np.float64)
    hi = (centre + 0.05).astype(np.float32).astype(np.float64)
    q = rng.standard_normal((1, d)).astype(np.float32).astype(np.float64)
    _, s = ref.unit_scores(q, hi, lo)
    mag = ref.score_magnitudes(q, hi, lo)
    terms = np.maximum(q * lo, q * hi).astype(np.float32)
    acc = np.zeros(len(s), dtype=np.float32)
    for j in range(d):
        acc = (acc + terms[:, j]).astype(np.float32)
    err = np.abs(acc.astype(np.float64) - s)
    assert np.all(err <= d * 2.0 ** -24 * mag)
    assert np.max(err / np.abs(s)) > 10 * np.max(err / mag)


def test_ambiguity_band_with_magnitudes():
    """Scores near zero with large magnitudes: the band is relative to the
    larger magnitude of the two pages, not to the k-th score."""
    s = np.array([10.0, 9.0, 1e-4, 0.0, -5.0])
    mag = np.array([10.0, 9.0, 200.0, 200.0, 5.0])
    amb, s_k = ref.ambiguous_pages(s, 5, 3, 0, 0)
    assert s_k == 1e-4 and amb == {2}
    amb, _ = ref.ambiguous_pages(s, 5, 3, 0, 0, mag=mag)
    assert amb == {2, 3}  # |0 - 1e-4| <= 1e-6 * 200
    amb, _ = ref.ambiguous_pages(s, 5, 3, 0, 0, rel=1e-7, mag=mag)
    assert amb == {2}
    # threshold band of the top-delta rule: scaled score 1e-4 against tau = 0
    # is decided either way only with the magnitude
    m = np.array([0.0])
    amb = ref.ambiguous_pages_topdelta(s, 5, 4, 1, 0, 1.0, m, 0.0)
    assert 2 not in amb
    amb = ref.ambiguous_pages_topdelta(s, 5, 4, 1, 0, 1.0, m, 0.0, mag=mag)
    assert 2 in amb and 3 in amb and 4 not in amb


def test_dense_is_exact_attention(small, tiny):
    check_dense_is_exact_attention(ref, small[2])
    check_dense_is_exact_attention(ref, tiny[1])


def test_restricted_reference_and_differs_from_dense(small, tiny):
    w, _, h = small
    differs = check_restricted_reference(ref, h, w.budget_pages, w.n_sink, w.n_local)
    assert differs > 1e-2
    differs = check_restricted_reference(ref, tiny[1], 8, 0, 0)
    assert differs > 1e-2


def test_sink():
    check_sink(ref)


def test_split_invariance():
    check_split_invariance(ref)


def test_split_ranges():
    check_split_ranges(ref)


def test_identical_heads_identical_rows():
    w, inp, h = small_inputs(needles=0)
    h = dict(h)
    q = h["q"].copy()
    q[:, 1] = q[:, 0]
    h["q"] = q
    res = ref.unit_step(h, 0, 0, w.budget_pages, w.n_sink, w.n_local)
    assert np.array_equal(res["out"][0], res["out"][1]) and res["lse"][0] == res["lse"][1]


def _relayout(h, perm):
    """Same logical content stored at permuted physical pages."""
    h2 = dict(h)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    h2["k_pool"] = h["k_pool"][inv]
    h2["v_pool"] = h["v_pool"][inv]
    table = h["page_table"].copy()
    for b in range(table.shape[0]):
        n = ref.num_pages(int(h["seq_lens"][b]), h["page_size"])
        table[b, :n] = perm[table[b, :n]]
    h2["page_table"] = table
    return h2


def check_pool_permutation(h, budget, n_sink, n_local, seed=3):
    perm = np.random.default_rng(seed).permutation(h["k_pool"].shape[0])
    h2 = _relayout(h, perm)
    for b in range(h["page_table"].shape[0]):
        for g in range(h["k_pool"].shape[1]):
            r1 = ref.unit_step(h, b, g, budget, n_sink, n_local)
            r2 = ref.unit_step(h2, b, g, budget, n_sink, n_local)
            assert np.array_equal(r1["scores"], r2["scores"])
            assert np.array_equal(r1["sel"], r2["sel"])
            assert np.array_equal(r1["out"], r2["out"])


def test_pool_permutation_invariance(small):
    w, _, h = small
    check_pool_permutation(h, w.budget_pages, w.n_sink, w.n_local)


def test_needles_are_found():
    # the needle recipe makes the needle pages score highest: with budget room
    # for all needles they are all kept (a property of the inputs, checked so
    # the workloads do what they claim)
    w, inp, h = small_inputs(needles=2, ctx_range=(400, 400), batch=1, head_dim=64,
                             budget_pages=6, max_pages=25)
    for g in range(w.num_kv_heads):
        res = ref.unit_step(h, 0, g, w.budget_pages, w.n_sink, w.n_local)
        assert set(inp["needle_pages"][(0, g)]) <= set(int(p) for p in res["sel"])


# ---------------------------------------------------------------------------
# Mutation tests: a planted mistake in the oracle must trip a pin.


def _expect_fail(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_mutation_score_drops_kmin_term(monkeypatch, small):
    def bad(q_group, kmax, kmin):
        u = (q_group[:, None, :] * kmax[None]).sum(-1)
        return u, u.max(0)
    monkeypatch.setattr(ref.pagesparse_ref, "unit_scores", bad)
    _expect_fail(check_score_admissible, ref.pagesparse_ref, small[2])


def test_mutation_score_min_instead_of_max(monkeypatch, small):
    def bad(q_group, kmax, kmin):
        u = np.minimum(q_group[:, None, :] * kmin[None], q_group[:, None, :] * kmax[None]).sum(-1)
        return u, u.max(0)
    monkeypatch.setattr(ref.pagesparse_ref, "unit_scores", bad)
    _expect_fail(check_score_admissible, ref.pagesparse_ref, small[2])


def test_mutation_group_sum_instead_of_max(monkeypatch):
    orig = ref.pagesparse_ref.unit_scores

    def bad(q_group, kmax, kmin):
        u, _ = orig(q_group, kmax, kmin)
        return u, u.sum(0)
    monkeypatch.setattr(ref.pagesparse_ref, "unit_scores", bad)
    _expect_fail(check_score_closed_forms, ref.pagesparse_ref)


def test_mutation_score_sign_flipped(monkeypatch):
    # (swapping the kmax and kmin arguments is not a mistake for this form:
    # the larger of the two products does not depend on their order)
    orig = ref.pagesparse_ref.unit_scores
    monkeypatch.setattr(ref.pagesparse_ref, "unit_scores",
                        lambda q, kmax, kmin: orig(-q, kmax, kmin))
    _expect_fail(check_score_closed_forms, ref.pagesparse_ref)


def test_mutation_meta_ignores_valid_mask(monkeypatch, small):
    def bad(k_pool, kv_dtype, page_table, seq_lens, b, g, page_size):
        n = ref.num_pages(int(seq_lens[b]), page_size)
        keys = np.stack([ref.widen(k_pool[int(page_table[b, p]), g], kv_dtype) for p in range(n)])
        return keys.max(1), keys.min(1)
    monkeypatch.setattr(ref.pagesparse_ref, "unit_page_meta", bad)
    _expect_fail(check_meta_bounds, ref.pagesparse_ref, small[2])


def test_mutation_meta_pool_ignores_valid_mask(monkeypatch, small):
    def bad(k_pool, kv_dtype, page_table, seq_lens, page_size, pages_of=None):
        out = {}
        for b in range(page_table.shape[0]):
            n = ref.num_pages(int(seq_lens[b]), page_size)
            pages = range(n) if pages_of is None else [p for p in pages_of[b] if 0 <= p < n]
            for p in pages:
                for g in range(k_pool.shape[1]):
                    keys = ref.widen(k_pool[int(page_table[b, p]), g], kv_dtype)
                    out[(int(page_table[b, p]), g)] = (keys.max(0), keys.min(0))
        return out
    monkeypatch.setattr(ref.pagesparse_ref, "page_meta_pool", bad)
    _expect_fail(check_meta_pool, ref.pagesparse_ref, small[2])


def test_mutation_meta_pool_ignores_pages_of(monkeypatch, small):
    orig = ref.pagesparse_ref.page_meta_pool
    monkeypatch.setattr(ref.pagesparse_ref, "page_meta_pool",
                        lambda k, dt, t, sl, ps, pages_of=None: orig(k, dt, t, sl, ps))
    _expect_fail(check_meta_pool, ref.pagesparse_ref, small[2])


def test_mutation_tie_to_higher_index(monkeypatch):
    def bad(scores, n, budget, n_sink, n_local):
        if budget >= n:
            return np.arange(n), list(range(n)), []
        forced = sorted(set(range(n_sink)) | set(range(n - n_local, n)))
        cand = np.array([p for p in range(n) if p not in forced])
        order = np.lexsort((-cand, -np.asarray(scores)[cand]))
        taken = [int(p) for p in cand[order[:budget - len(forced)]]]
        return np.array(sorted(set(forced) | set(taken))), forced, taken
    monkeypatch.setattr(ref.pagesparse_ref, "select_pages", bad)
    _expect_fail(check_selection_bruteforce, ref.pagesparse_ref)


def test_mutation_budget_excludes_forced(monkeypatch):
    orig = ref.pagesparse_ref.select_pages

    def bad(scores, n, budget, n_sink, n_local):
        f = len(set(range(min(n_sink, n))) | set(range(max(0, n - n_local), n)))
        return orig(scores, n, budget + f if budget < n else budget, n_sink, n_local)
    monkeypatch.setattr(ref.pagesparse_ref, "select_pages", bad)
    scores = np.random.default_rng(2).standard_normal(12)
    _expect_fail(check_selection_rank_count, ref.pagesparse_ref, scores, 12, 5, 1, 2)


def test_mutation_sink_in_numerator(monkeypatch):
    orig = ref.pagesparse_ref.attend

    def bad(q_h, keys, values, scale, sink=None):
        if sink is None or sink == -math.inf:
            return orig(q_h, keys, values, scale, None)
        k2 = np.vstack([keys, np.zeros((1, keys.shape[1]))])
        v2 = np.vstack([values, np.ones((1, values.shape[1]))])  # value not zero
        x = scale * (k2 @ q_h)
        x[-1] = sink
        m = x.max()
        w = np.exp(x - m)
        return (w @ v2) / w.sum(), m + math.log(w.sum())
    monkeypatch.setattr(ref.pagesparse_ref, "attend", bad)
    _expect_fail(check_sink, ref.pagesparse_ref)


def test_mutation_merge_without_rescale(monkeypatch):
    def bad(parts, sink=None):
        parts = [p for p in parts if p[0] != -math.inf]
        big_l = sum(l for _, l, _ in parts)
        acc = sum(a for _, _, a in parts)
        return acc / big_l, max(m for m, _, _ in parts) + math.log(big_l)
    monkeypatch.setattr(ref.pagesparse_ref, "combine_partials", bad)
    _expect_fail(check_split_invariance, ref.pagesparse_ref)


def test_mutation_scale_dropped(monkeypatch, tiny):
    orig = ref.pagesparse_ref.attend
    monkeypatch.setattr(ref.pagesparse_ref, "attend",
                        lambda q, k, v, scale, sink=None: orig(q, k, v, 1.0, sink))
    _expect_fail(check_dense_is_exact_attention, ref.pagesparse_ref, tiny[1])


def test_mutation_gather_ignores_page_table(monkeypatch, small):
    def bad(pool, kv_dtype, page_table, seq_lens, b, g, pages, page_size):
        rows = []
        for p in pages:
            cnt = ref.page_token_count(int(seq_lens[b]), int(p), page_size)
            rows.append(ref.widen(pool[int(p), g, :cnt], kv_dtype))  # logical id used as physical
        return np.concatenate(rows) if rows else np.zeros((0, pool.shape[-1]))
    monkeypatch.setattr(ref.pagesparse_ref, "gather_tokens", bad)
    w, _, h = small
    _expect_fail(check_pool_permutation, h, w.budget_pages, w.n_sink, w.n_local)


def test_mutation_fp8_round_to_nearest(monkeypatch):
    t = ref.fp8_e4m3_table()

    def nearest(x):
        fin = np.array([c for c in range(256) if not math.isnan(t[c]) and c != 0x80])
        x = np.asarray(x, dtype=np.float64)
        return fin[np.abs(t[fin][None, :] - x.reshape(-1, 1)).argmin(1)].astype(np.uint8).reshape(
            x.shape)
    monkeypatch.setattr(ref.pagesparse_ref, "fp8_round_up", nearest)
    _expect_fail(check_fp8_directed_rounding, ref.pagesparse_ref)


def test_mutation_fp8_exponent_bias(monkeypatch):
    orig = ref.pagesparse_ref.fp8_e4m3_value
    monkeypatch.setattr(ref.pagesparse_ref, "fp8_e4m3_value", lambda c: 2.0 * orig(c))
    _expect_fail(check_fp8_decode, ref.pagesparse_ref)


def test_mutation_fp8_signed_zero_code(monkeypatch):
    orig = ref.pagesparse_ref.fp8_round_up

    def bad(x):
        c = np.array(orig(x))
        c[(c == 0) & (np.asarray(x) < 0)] = 0x80
        return c
    monkeypatch.setattr(ref.pagesparse_ref, "fp8_round_up", bad)
    _expect_fail(check_fp8_directed_rounding, ref.pagesparse_ref)


def test_mutation_topdelta_max_over_heads(monkeypatch):
    """Taking the largest pseudo-max of the group (instead of the smallest)
    drops pages some head needs."""
    orig = ref.pagesparse_ref.select_pages_topdelta

    def bad(scores, n, budget, n_sink, n_local, scale, m_tilde, delta):
        return orig(scores, n, budget, n_sink, n_local, scale,
                    np.full_like(m_tilde, np.max(m_tilde)), delta)
    monkeypatch.setattr(ref.pagesparse_ref, "select_pages_topdelta", bad)
    w, _, h = tight_small_inputs(2)
    _expect_fail(check_topdelta, ref.pagesparse_ref, h, w)


def test_mutation_topdelta_unscaled_bound(monkeypatch):
    orig = ref.pagesparse_ref.select_pages_topdelta
    monkeypatch.setattr(ref.pagesparse_ref, "select_pages_topdelta",
                        lambda s, n, bu, ns, nl, sc, mt, d: orig(s, n, bu, ns, nl, 1.0, mt, d))
    w, _, h = tight_small_inputs()
    _expect_fail(check_topdelta, ref.pagesparse_ref, h, w)
