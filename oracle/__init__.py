"""CPU fp64 oracle for page-selected sparse decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The product path (the HIP library and its Python binding) never
imports it, and this package never imports the product path.
"""

from .pagesparse_ref import (  # noqa: F401
    BF16,
    F32,
    AMBIGUITY_REL,
    widen,
    num_pages,
    page_token_count,
    unit_page_meta,
    page_meta_pool,
    unit_scores,
    score_magnitudes,
    FP8_E4M3,
    FP8_MAX,
    fp8_e4m3_value,
    fp8_e4m3_table,
    fp8_round_up,
    fp8_round_down,
    widen_fp8,
    fp8_bounds,
    select_pages,
    pseudo_max,
    select_pages_topdelta,
    ambiguous_pages_topdelta,
    ambiguous_pages,
    gather_tokens,
    attend,
    split_partial,
    combine_partials,
    sparse_split_slots,
    dense_split_pages,
    unit_step,
    full_decode,
)
