"""Plain, slow, fp64 reference of query-aware page-selected sparse decode.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path. It shares
no code with the HIP library; the only thing both sides use is the seeded
input generator in ``workloads/``, which holds none of the arithmetic below.

Sources (cited by page title and section):

* "Don't read the haystack", section "Part two: the skipping": per page keep
  the elementwise min and max of its keys; the page bound is the sum over d of
  the larger of q_d*kmin_d and q_d*kmax_d, which upper-bounds every q.k in the
  page; pages are ranked by the bound, the top k are kept together with the
  sink page and the last few local pages, and a sparse twin of the dense
  decode walks that page list.
* Same page, section "Part one: hitting the wall on purpose": split-KV
  flash-decoding; each split writes running max, normaliser and unnormalised
  accumulator in fp32, and a second stage merges them with the log-sum-exp
  rescale. Contexts need not be multiples of anything.
* "Attention: Undivided & Uncompressed", section "Traffic": the online
  softmax merge of two partial softmaxes by rescaling with exp(m1 - m2), whose
  result equals the full-row softmax exactly.
* "Training-free sparse attention for long-context LLM decode", section
  "Strongest signals", item 1: a learned per-head sink logit enters only the
  softmax denominator, as a virtual key whose value vector is zero.
* "perf(core): fused sparse-attention decode via page indirection - #1005",
  sections "The reduction, and why it needed no kernel change" (a token is
  reached through a page list that need not be adjacent or ordered; one KV
  head owns its group of query heads) and "Making the selection inspectable
  and proving it against dense" (output equals a reference restricted to the
  selected positions).

Readings taken where the pages are silent:

1. GQA: one page list per (request, KV head); the group's score for a page
   is the MAX over the group's query heads of the per-head bound. No page says
   how heads combine; the max keeps the bound admissible for every head of the
   group. Parity unpinned by the pages (pinned only to this reading).
2. The budget counts the forced pages: a request with n pages keeps
   min(budget, n) pages; top-k fills budget - |forced|. Parity unpinned by
   the pages (pinned only to this reading).
3. Ties between equal scores go to the lower logical page index; the page
   list is emitted in ascending logical order.
4. The bound is unscaled (a positive scale does not change the ranking).
5. The sink logit is in the same natural-log units as scale*q.k, is not
   multiplied by scale, and takes no part in page selection.
6. Only valid tokens (t < seq_len) enter metadata and attention.

Precision: every input is fp32 or bf16. bf16 is widened exactly (its bits
are the high half of an fp32). Products fp32*bf16 (24+8 bits) and fp32*fp32
(48 bits) are exact in fp64's 53-bit significand, so the only rounding here is
fp64 summation, exp and log.
"""

from __future__ import annotations

import math

import numpy as np

BF16 = "bf16"
F32 = "f32"

#: Relative band around the k-th selected score inside which the choice
#: between pages is reported as ambiguous instead of being required to match.
#: Relative to the score itself, or, when the page magnitudes are given
#: (score_magnitudes), to the larger magnitude of the two pages compared: a
#: sum of D terms rounded in fp32 is off by at most about D * 2^-24 times the
#: sum of the terms' absolute values (the forward error bound of recursive
#: summation), which is far above the result when the terms cancel.
AMBIGUITY_REL = 1e-6


# ---------------------------------------------------------------------------
# Storage


def widen(a: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Exact float64 value of stored K/V/meta elements.

    bf16 arrives as its raw 16-bit patterns (uint16); its value is the fp32
    whose high 16 bits are those bits and whose low 16 bits are zero.
    """
    if kv_dtype == BF16:
        a = np.asarray(a)
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if kv_dtype == F32:
        a = np.asarray(a)
        if a.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def num_pages(seq_len: int, page_size: int) -> int:
    """Pages a context of seq_len tokens occupies: ceil(seq_len / page_size).

    "Attention: Undivided & Uncompressed", section "Bytes": a paged cache
    allocates ceil(n/B) pages, so at most one page per sequence is partial.
    """
    if seq_len < 0 or page_size <= 0:
        raise ValueError("seq_len must be >= 0 and page_size > 0")
    return -(-int(seq_len) // int(page_size))


def page_token_count(seq_len: int, p: int, page_size: int) -> int:
    """Valid tokens on logical page p: those t with p*P <= t < min((p+1)*P, len)."""
    return max(0, min(page_size, int(seq_len) - p * page_size))


# ---------------------------------------------------------------------------
# Stage 1: page metadata ("Don't read the haystack", "Part two: the skipping")


def unit_page_meta(k_pool, kv_dtype, page_table, seq_lens, b, g, page_size):
    """Elementwise max and min of the valid keys of each logical page.

    Returns (kmax, kmin), each float64 [n_pages(b), D], for request b and KV
    head g. Slots past the sequence end on the last page are ignored. The
    full pages are reduced together (their token axis is whole); the last
    page, which may be partial, is reduced over its valid tokens only.
    """
    seq_len = int(seq_lens[b])
    n = num_pages(seq_len, page_size)
    d = k_pool.shape[-1]
    kmax = np.empty((n, d), dtype=np.float64)
    kmin = np.empty((n, d), dtype=np.float64)
    if n == 0:
        return kmax, kmin
    phys = np.asarray(page_table[b, :n], dtype=np.int64)
    if n > 1:  # pages 0 .. n-2 hold page_size valid tokens each
        keys = widen(np.asarray(k_pool[phys[:-1], g]), kv_dtype)  # [n-1, page, D]
        kmax[:-1] = keys.max(axis=1)
        kmin[:-1] = keys.min(axis=1)
    cnt = page_token_count(seq_len, n - 1, page_size)
    last = widen(np.asarray(k_pool[phys[-1], g, :cnt, :]), kv_dtype)  # [cnt, D]
    kmax[-1] = last.max(axis=0)
    kmin[-1] = last.min(axis=0)
    return kmax, kmin


def page_meta_pool(k_pool, kv_dtype, page_table, seq_lens, page_size, pages_of=None):
    """Metadata for every mapped physical page, as {(phys, g): (kmax, kmin)}.

    pages_of: optional {b: iterable of logical pages} restricting the build
    (used for the incremental tail-page update). Physical pages no request
    maps are absent from the result.
    """
    out = {}
    hkv = k_pool.shape[1]
    for b in range(page_table.shape[0]):
        n = num_pages(int(seq_lens[b]), page_size)
        pages = range(n) if pages_of is None else [p for p in pages_of[b] if 0 <= p < n]
        for p in pages:
            phys = int(page_table[b, p])
            cnt = page_token_count(int(seq_lens[b]), p, page_size)
            for g in range(hkv):
                keys = widen(k_pool[phys, g, :cnt, :], kv_dtype)
                out[(phys, g)] = (keys.max(axis=0), keys.min(axis=0))
    return out


# ---------------------------------------------------------------------------
# Stage 2: the page bound ("Don't read the haystack", "Part two: the skipping")


def unit_scores(q_group: np.ndarray, kmax: np.ndarray, kmin: np.ndarray):
    """Per-head bounds U[h, p] and the group score S[p] = max_h U[h, p].

    U[h, p] = sum_d max(q[h,d]*kmin[p,d], q[h,d]*kmax[p,d]), the larger of the
    two products for each coordinate, so U >= q.k for every key in the page.
    q_group: float64 [G, D] (the query heads sharing this KV head).
    """
    q = np.asarray(q_group, dtype=np.float64)
    prod_min = q[:, None, :] * kmin[None, :, :]  # [G, n, D]
    prod_max = q[:, None, :] * kmax[None, :, :]
    u = np.maximum(prod_min, prod_max).sum(axis=-1)  # [G, n]
    return u, u.max(axis=0)


def score_magnitudes(q_group: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """Per page, the largest over the group's heads of the sum of the absolute
    values of the D terms of U[h, p]: the scale of the rounding error of any
    fp32 evaluation of the score (never below |S[p]|)."""
    q = np.asarray(q_group, dtype=np.float64)
    terms = np.maximum(q[:, None, :] * kmin[None, :, :], q[:, None, :] * kmax[None, :, :])
    return np.abs(terms).sum(axis=-1).max(axis=0)


# ---------------------------------------------------------------------------
# Stage 1-2 variant: compressed metadata (8-bit bounds)
#
# "Faster Than Flash: Exploiting Attention Sparsity for Efficient Long-Context
# Decoding", section "Methodology", item 1 (content-aware scanning via
# low-bit quantization): the scan that decides which blocks to read runs on a
# low-bit copy, and the kept blocks are then read at full precision. Applied
# here to the page metadata, the stream that dominates the scan, with the
# rounding directed so that the bound of "Don't read the haystack" ("Part
# two: the skipping") stays an upper bound: kmax is rounded up and kmin down,
# so the 8-bit box contains the exact one and, for every q, the bound can only
# grow. The attention itself still reads the full-precision keys and values.
#
# Format (a reading: the pages name no 8-bit format): the 8-bit
# floating point E4M3 of the OCP 8-bit floating point specification, the
# variant without infinities: 1 sign bit, 4 exponent bits with bias 7, 3
# mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the two
# codes with every exponent and mantissa bit set are NaN; the largest finite
# magnitude is 448. A zero result is always code 0x00. A bound beyond +-448
# saturates to +-448 (the fp8 metadata mode requires |K| <= 448; beyond it the
# saturated bound is no longer admissible).

FP8_E4M3 = "fp8_e4m3"
FP8_MAX = 448.0


def fp8_e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the format's definition (NaN codes give nan)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_table() -> np.ndarray:
    """float64 [256]: the value of every code."""
    return np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def _fp8_finite_sorted():
    """(values ascending, their codes) over the finite codes, one code per
    value (zero is 0x00)."""
    t = fp8_e4m3_table()
    by_val = {}
    for c in range(256):
        v = t[c]
        if math.isnan(v):
            continue
        if v == 0.0:
            c = 0x00
        by_val.setdefault(v, c)
    vals = np.array(sorted(by_val), dtype=np.float64)
    return vals, np.array([by_val[v] for v in vals], dtype=np.uint8)


def fp8_round_up(x) -> np.ndarray:
    """Code of the smallest finite E4M3 value >= x (saturating at 448)."""
    vals, codes = _fp8_finite_sorted()
    x = np.asarray(x, dtype=np.float64)
    i = np.searchsorted(vals, x, side="left")
    return codes[np.minimum(i, len(vals) - 1)]


def fp8_round_down(x) -> np.ndarray:
    """Code of the largest finite E4M3 value <= x (saturating at -448)."""
    vals, codes = _fp8_finite_sorted()
    x = np.asarray(x, dtype=np.float64)
    i = np.searchsorted(vals, x, side="right") - 1
    return codes[np.maximum(i, 0)]


def widen_fp8(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8)."""
    return fp8_e4m3_table()[np.asarray(codes, dtype=np.uint8)]


def fp8_bounds(kmax: np.ndarray, kmin: np.ndarray):
    """The 8-bit metadata of exact bounds: (codes of kmax rounded up, codes of
    kmin rounded down), uint8 arrays of the input shapes."""
    return fp8_round_up(kmax), fp8_round_down(kmin)


# ---------------------------------------------------------------------------
# Stage 3: selection


def _forced(n: int, n_sink: int, n_local: int):
    return sorted(set(range(min(n_sink, n))) | set(range(max(0, n - n_local), n)))


def select_pages(scores: np.ndarray, n: int, budget: int, n_sink: int, n_local: int):
    """Logical pages kept for one (request, KV head), ascending.

    If the budget covers all n pages every page is kept (the dense case).
    Otherwise the first n_sink and last n_local pages are always kept and the
    remaining budget - |forced| slots go to the other pages in order of
    decreasing score, ties to the lower page index.
    Returns (sel: int64 array ascending, forced: list, taken: list of the
    scored pages in the order they were taken).
    """
    if budget >= n:
        return np.arange(n, dtype=np.int64), list(range(n)), []
    forced = _forced(n, n_sink, n_local)
    r = budget - len(forced)
    if r < 0:
        raise ValueError("forced pages exceed the budget")
    fset = set(forced)
    cand = np.array([p for p in range(n) if p not in fset], dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)[cand]
    order = np.lexsort((cand, -s))  # primary: score descending; then index ascending
    taken = [int(p) for p in cand[order[:r]]]
    sel = np.array(sorted(fset | set(taken)), dtype=np.int64)
    return sel, forced, taken


def _band(s, k, mag, rel):
    """Per page, the half-width of the band around page k's score: rel*|s_k|,
    or rel*max(mag[p], mag[k]) with the page magnitudes."""
    if mag is None:
        return np.full(len(s), rel * abs(float(s[k])))
    m = np.asarray(mag, dtype=np.float64)
    return rel * np.maximum(m[:len(s)], m[k])


def ambiguous_pages(scores, n, budget, n_sink, n_local, rel=AMBIGUITY_REL, mag=None):
    """Scored pages whose score lies within the band (rel*|s_k|, or relative
    to the page magnitudes mag when given) of the k-th taken score s_k.

    A page choice inside this set may legitimately differ between an fp32
    device and this fp64 reference. Returns (set, s_k or None).
    """
    sel, forced, taken = select_pages(scores, n, budget, n_sink, n_local)
    if not taken:
        return set(), None
    s = np.asarray(scores, dtype=np.float64)
    k = taken[-1]
    s_k = float(s[k])
    band = _band(s, k, mag, rel)
    fset = set(forced)
    amb = {p for p in range(n) if p not in fset and abs(s[p] - s_k) <= band[p]}
    return amb, s_k


# ---------------------------------------------------------------------------
# Stage 3 variant: top-delta threshold selection
#
# "Faster Than Flash: Exploiting Attention Sparsity for Efficient Long-Context
# Decoding", section "Methodology", item 2 (Top-delta selection criterion),
# eq. (1)-(3) and section "Pseudo-Max Robustness as Fail-Safe": a block is
# kept when its logit is at least the row maximum minus delta; the maximum is
# replaced by a pseudo-max taken over the sink and local tokens only, which is
# never larger, so the kept set can only grow. Readings for a page list
# shared by a group of query heads, scored by the page bound:
# * the pseudo-max of head h is the largest scale*q_h.k_t over the valid
#   tokens of the forced pages (the first n_sink and last n_local pages); with
#   no forced page there is no pseudo-max and the threshold is -inf;
# * the group threshold is the smallest of its heads' pseudo-maxima minus
#   delta, so that the list keeps, for every head, every page the per-head
#   criterion would keep;
# * a page passes when scale*S(p) >= threshold (S the group's bound, which is
#   >= every q_h.k_t of the page), so every token passing the criterion with
#   the true maximum lies on a kept page;
# * the count is capped at the budget to stay graph-capturable: the forced
#   pages and then the passing pages by decreasing score (ties to the lower
#   page), at most budget - |forced| of them.


def pseudo_max(q_group: np.ndarray, keys_forced: np.ndarray, scale: float) -> np.ndarray:
    """Per query head, max over the forced tokens of scale * q_h . k_t
    ([FFD] eq. (3)); -inf for every head when there is no forced token."""
    q = np.asarray(q_group, dtype=np.float64)
    if keys_forced.shape[0] == 0:
        return np.full(q.shape[0], -np.inf)
    return (float(scale) * (q @ np.asarray(keys_forced, dtype=np.float64).T)).max(axis=1)


def select_pages_topdelta(scores, n, budget, n_sink, n_local, scale, m_tilde, delta):
    """Kept pages of one (request, KV head) under the top-delta criterion.

    Returns (sel ascending, forced, taken in the order taken, threshold).
    With budget >= n every page is kept (threshold None).
    """
    if budget >= n:
        return np.arange(n, dtype=np.int64), list(range(n)), [], None
    forced = _forced(n, n_sink, n_local)
    r = budget - len(forced)
    if r < 0:
        raise ValueError("forced pages exceed the budget")
    tau = float(np.min(m_tilde)) - float(delta) if len(forced) else -math.inf
    fset = set(forced)
    s = np.asarray(scores, dtype=np.float64)
    cand = np.array([p for p in range(n) if p not in fset and float(scale) * s[p] >= tau],
                    dtype=np.int64)
    order = np.lexsort((cand, -s[cand])) if len(cand) else np.array([], dtype=np.int64)
    taken = [int(p) for p in cand[order[:r]]]
    sel = np.array(sorted(fset | set(taken)), dtype=np.int64)
    return sel, forced, taken, tau


def ambiguous_pages_topdelta(scores, n, budget, n_sink, n_local, scale, m_tilde, delta,
                             rel=AMBIGUITY_REL, mag=None):
    """Pages an fp32 device may decide differently: scaled scores within
    rel of the threshold (it is itself an fp32 result on the device; with the
    page magnitudes mag, within rel times the larger of |tau|, 1 and the
    page's scaled magnitude), and, when the cap binds, scores within the band
    of ambiguous_pages around the last taken one."""
    sel, forced, taken, tau = select_pages_topdelta(scores, n, budget, n_sink, n_local, scale,
                                                    m_tilde, delta)
    if tau is None:
        return set()
    s = np.asarray(scores, dtype=np.float64)
    fset = set(forced)
    amb = set()
    if math.isfinite(tau):
        m = np.zeros(n) if mag is None else float(scale) * np.asarray(mag, dtype=np.float64)
        amb |= {p for p in range(n) if p not in fset and
                abs(float(scale) * s[p] - tau) <= rel * max(abs(tau), 1.0, m[p])}
    r = budget - len(forced)
    if taken and len(taken) == r:
        k = taken[-1]
        band = _band(s, k, mag, rel)
        amb |= {p for p in range(n) if p not in fset and abs(s[p] - s[k]) <= band[p]}
    return amb


# ---------------------------------------------------------------------------
# Stage 4: attention over the kept tokens


def gather_tokens(pool, kv_dtype, page_table, seq_lens, b, g, pages, page_size):
    """float64 rows [T, D] of the valid tokens on the given logical pages."""
    rows = []
    for p in pages:
        phys = int(page_table[b, int(p)])
        cnt = page_token_count(int(seq_lens[b]), int(p), page_size)
        rows.append(widen(pool[phys, g, :cnt, :], kv_dtype))
    if not rows:
        return np.zeros((0, pool.shape[-1]), dtype=np.float64)
    return np.concatenate(rows, axis=0)


def attend(q_h, keys, values, scale, sink=None):
    """Softmax attention of one query over given keys, with an optional sink.

    x_t = scale * (q . k_t). The sink logit s joins only the normaliser, as a
    key whose value vector is zero ("Training-free sparse attention for
    long-context LLM decode", "Strongest signals", item 1):
        M = max(max_t x_t, s);  Z = sum_t e^(x_t - M) + e^(s - M)
        out = sum_t e^(x_t - M) v_t / Z;  lse = M + ln Z.
    Plain two-pass evaluation, no online rescaling and no splits.
    Returns (out float64 [D], lse float).
    """
    x = float(scale) * (keys @ np.asarray(q_h, dtype=np.float64))
    s = -math.inf if sink is None else float(sink)
    m = max(float(x.max()) if x.size else -math.inf, s)
    if m == -math.inf:
        return np.zeros(values.shape[-1]), -math.inf
    w = np.exp(x - m)
    z = float(w.sum()) + (math.exp(s - m) if s != -math.inf else 0.0)
    return (w @ values) / z, m + math.log(z)


def split_partial(q_h, keys, values, scale):
    """Partial softmax state of one KV slice ("Part one": running max, normaliser,
    unnormalised accumulator). An empty slice gives (-inf, 0, zeros)."""
    if keys.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(values.shape[-1])
    x = float(scale) * (keys @ np.asarray(q_h, dtype=np.float64))
    m = float(x.max())
    w = np.exp(x - m)
    return m, float(w.sum()), w @ values


def combine_partials(parts, sink=None):
    """Log-sum-exp merge of split partials, with the sink as one more partial
    (m = s, l = 1, acc = 0) ("Attention: Undivided & Uncompressed", "Traffic").

    parts: iterable of (m, l, acc). Returns (out, lse).
    """
    parts = list(parts)
    if sink is not None and float(sink) != -math.inf:
        parts.append((float(sink), 1.0, np.zeros_like(parts[0][2])))
    big_m = max(m for m, _, _ in parts)
    if big_m == -math.inf:
        return np.zeros_like(parts[0][2]), -math.inf
    big_l = 0.0
    acc = np.zeros_like(parts[0][2])
    for m, l, a in parts:
        if m == -math.inf:
            continue
        w = math.exp(m - big_m)
        big_l += w * l
        acc = acc + w * a
    return acc / big_l, big_m + math.log(big_l)


def sparse_split_slots(budget: int, n_splits: int):
    """Slots [lo, hi) of the kept-page list that split s covers: chunks of
    ceil(budget / n_splits) slots. Slots past the kept count are empty."""
    c = -(-budget // n_splits)
    return [(min(s * c, budget), min((s + 1) * c, budget)) for s in range(n_splits)]


def dense_split_pages(n: int, n_splits: int):
    """Logical pages [lo, hi) that split s of the dense decode covers:
    chunks of ceil(n / n_splits) pages of this request."""
    c = -(-n // n_splits)
    return [(min(s * c, n), min((s + 1) * c, n)) for s in range(n_splits)]


# ---------------------------------------------------------------------------
# Whole step


def unit_step(inp, b, g, budget, n_sink, n_local, sel_override=None, delta=None):
    """Score, select and attend for one (request b, KV head g).

    inp: dict of host arrays with keys q [B,Hq,D] f32, k_pool, v_pool,
    kv_dtype, page_table, seq_lens, page_size, scale (the fp32 value the
    device uses), sink ([Hq] f32 or None), and optionally meta_format
    (FP8_E4M3: pages are scored on the 8-bit bounds).
    sel_override: attend over this page list instead of the selected one.
    delta: select by the top-delta criterion with this delta (None: top-k).
    Returns a dict with u, scores, mag (score_magnitudes), sel, forced, taken,
    out [G,D], lse [G].
    """
    q = inp["q"]
    hq, hkv = q.shape[1], inp["k_pool"].shape[1]
    grp = hq // hkv
    ps = inp["page_size"]
    n = num_pages(int(inp["seq_lens"][b]), ps)
    kmax, kmin = unit_page_meta(inp["k_pool"], inp["kv_dtype"], inp["page_table"],
                                inp["seq_lens"], b, g, ps)
    if inp.get("meta_format") == FP8_E4M3:  # the scan reads the 8-bit bounds
        cmax, cmin = fp8_bounds(kmax, kmin)
        kmax, kmin = widen_fp8(cmax), widen_fp8(cmin)
    qg = q[b, g * grp:(g + 1) * grp].astype(np.float64)
    u, s = unit_scores(qg, kmax, kmin)
    mag = score_magnitudes(qg, kmax, kmin)
    tau = None
    if delta is None:
        sel, forced, taken = select_pages(s, n, budget, n_sink, n_local)
    else:  # top-delta: the pseudo-max over the forced pages' tokens
        fpages = _forced(n, n_sink, n_local) if budget < n else []
        kf = gather_tokens(inp["k_pool"], inp["kv_dtype"], inp["page_table"], inp["seq_lens"],
                           b, g, fpages, ps)
        m_tilde = pseudo_max(qg, kf, inp["scale"])
        sel, forced, taken, tau = select_pages_topdelta(s, n, budget, n_sink, n_local,
                                                        inp["scale"], m_tilde, delta)
    pages = sel if sel_override is None else np.asarray(sel_override, dtype=np.int64)
    keys = gather_tokens(inp["k_pool"], inp["kv_dtype"], inp["page_table"], inp["seq_lens"],
                         b, g, pages, ps)
    vals = gather_tokens(inp["v_pool"], inp["kv_dtype"], inp["page_table"], inp["seq_lens"],
                         b, g, pages, ps)
    outs, lses = [], []
    for i in range(grp):
        h = g * grp + i
        sk = None if inp.get("sink") is None else inp["sink"][h]
        o, l = attend(qg[i], keys, vals, inp["scale"], sk)
        outs.append(o)
        lses.append(l)
    return {"u": u, "scores": s, "mag": mag, "sel": sel, "forced": forced, "taken": taken,
            "out": np.stack(outs), "lse": np.array(lses), "n": n, "tau": tau}


def full_decode(inp, b, h):
    """Exact softmax attention of query head h of request b over every valid
    token (the dense decode; with the sink folded in when present)."""
    q = inp["q"]
    hq, hkv = q.shape[1], inp["k_pool"].shape[1]
    g = h // (hq // hkv)
    n = num_pages(int(inp["seq_lens"][b]), inp["page_size"])
    pages = range(n)
    keys = gather_tokens(inp["k_pool"], inp["kv_dtype"], inp["page_table"], inp["seq_lens"],
                         b, g, pages, inp["page_size"])
    vals = gather_tokens(inp["v_pool"], inp["kv_dtype"], inp["page_table"], inp["seq_lens"],
                         b, g, pages, inp["page_size"])
    sk = None if inp.get("sink") is None else inp["sink"][h]
    return attend(q[b, h].astype(np.float64), keys, vals, inp["scale"], sk)
