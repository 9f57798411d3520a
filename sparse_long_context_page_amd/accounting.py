"""Host-side byte accounting of a decode step (no device work).

The roofline of this path counts algorithmic bytes only: the per-page min/max
metadata of every page of every (request, KV head) plus the K and V rows of
the valid tokens on the kept pages. A dense decode reads every valid K and V
row. ("Don't read the haystack", sections "Why generating a token is a
reading problem" and "Part two: the skipping"; "Attention: Undivided &
Uncompressed", section "Bytes": a paged cache charges ceil(n/B) pages.)
"""

from __future__ import annotations

from typing import Iterable, Sequence


def pages_for(tokens: int, page_size: int) -> int:
    """ceil(tokens / page_size)."""
    if tokens < 0 or page_size <= 0:
        raise ValueError("tokens must be >= 0 and page_size > 0")
    return -(-int(tokens) // int(page_size))


def paged_waste(tokens: int, page_size: int) -> float:
    """Allocated slots per live token of a paged cache, ceil(n/B)*B/n."""
    return pages_for(tokens, page_size) * page_size / tokens


def slab_waste(slab_tokens: int, tokens: int) -> float:
    """Allocated slots per live token of a contiguous reservation."""
    return slab_tokens / tokens


def meta_bytes(seq_lens: Sequence[int], kv_heads: int, head_dim: int, elem_bytes: int,
               page_size: int) -> int:
    """Bytes of (kmax, kmin) over every page of every (request, KV head)."""
    return sum(pages_for(n, page_size) for n in seq_lens) * kv_heads * 2 * head_dim * elem_bytes


def meta_fraction_of_keys(page_size: int) -> float:
    """Metadata size relative to the key cache: 2 vectors per page of page_size keys."""
    return 2.0 / page_size


def kept_tokens(seq_len: int, kept_pages: Iterable[int], page_size: int) -> int:
    """Valid tokens on the given logical pages of one request."""
    return sum(max(0, min(page_size, seq_len - p * page_size)) for p in kept_pages)


def selected_kv_bytes_uniform(seq_lens: Sequence[int], kv_heads: int, head_dim: int,
                              elem_bytes: int, page_size: int, budget_pages: int) -> int:
    """K+V bytes of the kept pages when every kept page is full except
    possibly the request's last page, which is always kept when it is partial
    (true whenever the last page is forced or the budget covers every page).
    For an exact figure use selected_kv_bytes with the actual page lists."""
    total = 0
    for n in seq_lens:
        np_ = pages_for(n, page_size)
        k = min(budget_pages, np_)
        last = n - (np_ - 1) * page_size
        toks = (k - 1) * page_size + last if k == np_ else k * page_size
        total += toks
    return total * kv_heads * 2 * head_dim * elem_bytes


def selected_kv_bytes(seq_lens: Sequence[int], page_lists, head_dim: int, elem_bytes: int,
                      page_size: int) -> int:
    """Exact K+V bytes of the kept pages: page_lists[(b, g)] = kept logical pages."""
    total = 0
    for (b, _g), pages in page_lists.items():
        total += kept_tokens(int(seq_lens[b]), [p for p in pages if p >= 0], page_size)
    return total * 2 * head_dim * elem_bytes


def dense_kv_bytes(seq_lens: Sequence[int], kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K+V bytes of every valid token."""
    return sum(int(n) for n in seq_lens) * kv_heads * 2 * head_dim * elem_bytes
