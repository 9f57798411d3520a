"""One decode step on the device: the stages of the C ABI in order.

DecodeStep owns the intermediate buffers of a fixed geometry (scores, page
lists, split partials, output), so a step allocates nothing and can be
captured into a HIP graph. The path taken is reported by name: "sparse"
(score -> select -> sparse decode -> combine, with select and sparse decode
in one launch where the fused entry point supports the geometry) or "dense"
(full decode -> combine), chosen on the host from the host-known context
lengths: when the
budget covers every page of every request, the dense decode is the same
computation with less work ("Don't read the haystack", section "Part two:
the skipping").
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import ops
from .ops import Geometry


class DecodeStep:
    def __init__(self, geom: Geometry, budget_pages: int, n_sink: int = 0, n_local: int = 0,
                 n_splits: int = 8, dense_splits: int = 32, scale: Optional[float] = None,
                 device="cuda", fused: bool = True, delta: Optional[float] = None,
                 merge_in_launch: bool = True):
        self.g = geom
        self.budget = int(budget_pages)
        self.n_sink = int(n_sink)
        self.n_local = int(n_local)
        self.n_splits = int(min(n_splits, self.budget))
        self.dense_splits = int(min(dense_splits, geom.max_pages))
        self.scale = ops.default_scale(geom.head_dim) if scale is None else float(scale)
        # top-delta selection (ps_select_topdelta) instead of top-k when set
        self.delta = None if delta is None else float(delta)
        # selection (top-k, or top-delta) fused into the sparse decode (one
        # launch) when supported
        self.fused = (bool(fused) and
                      ops.select_decode_supported(geom, self.budget, self.n_splits))
        # with several splits, the fused launch also merges them (the last
        # split of each (request, KV head) to finish), counting arrivals in a
        # zeroed [B, Hkv] buffer that every launch leaves zeroed
        self.merge_in_launch = self.fused and bool(merge_in_launch)
        self.arrivals = (torch.zeros((geom.batch, geom.num_kv_heads), device=device,
                                     dtype=torch.int32) if self.merge_in_launch else None)
        b, hq, hkv, d = geom.batch, geom.num_q_heads, geom.num_kv_heads, geom.head_dim
        f32 = dict(device=device, dtype=torch.float32)
        self.scores = torch.empty((b, hkv, geom.max_pages), **f32)
        self.sel = torch.empty((b, hkv, self.budget), device=device, dtype=torch.int32)
        self.sel_count = torch.empty((b, hkv), device=device, dtype=torch.int32)
        s_max = max(self.n_splits, self.dense_splits)
        self._acc = torch.empty((b * hq * s_max * d,), **f32)
        self._ml = torch.empty((b * hq * s_max * 2,), **f32)
        self.out = torch.empty((b, hq, d), **f32)
        self.lse = torch.empty((b, hq), **f32)

    def partials(self, n_splits: int):
        g = self.g
        n = g.batch * g.num_q_heads * n_splits
        return (self._acc[:n * g.head_dim].view(g.batch, g.num_q_heads, n_splits, g.head_dim),
                self._ml[:n * 2].view(g.batch, g.num_q_heads, n_splits, 2))

    def path_for(self, seq_lens_host: Sequence[int]) -> str:
        n_max = max((int(x) + self.g.page_size - 1) // self.g.page_size for x in seq_lens_host)
        return "dense" if self.budget >= n_max else "sparse"

    def refresh_tail_meta(self, k_pool, page_table, seq_lens, tail_begin, meta, stream=None):
        """Rebuild the metadata of each request's last page (the page a decode
        step appends to); tail_begin[b] = n_b - 1."""
        ops.ps_build_page_meta(self.g, k_pool, page_table, seq_lens, tail_begin, 1, meta, stream)

    def sparse(self, q, k_pool, v_pool, meta, page_table, seq_lens, sink=None, stream=None,
               refresh_tail=False):
        """Score, select, decode and merge. With refresh_tail the metadata of
        each request's last page is rebuilt inside the score launch
        (ps_refresh_score_pages)."""
        g = self.g
        if refresh_tail:
            ops.ps_refresh_score_pages(g, q, k_pool, meta, page_table, seq_lens, self.scores,
                                       stream)
        else:
            ops.ps_score_pages(g, q, meta, page_table, seq_lens, self.scores, stream)
        acc, ml = self.partials(self.n_splits)
        if self.fused:
            head = (g, q, k_pool, v_pool, page_table, seq_lens, self.scores, self.budget,
                    self.n_sink, self.n_local, self.scale)
            if self.delta is None:
                fn = ops.ps_select_sparse_decode
            else:
                fn = ops.ps_select_topdelta_sparse_decode
                head = head + (self.delta,)
            if self.n_splits == 1:  # select, decode and merge in one launch
                fn(*head, 1, self.sel, self.sel_count, None, None, sink, self.out, self.lse,
                   stream)
                return self.out, self.lse
            if self.merge_in_launch:  # the last split to finish merges
                fn(*head, self.n_splits, self.sel, self.sel_count, acc, ml, sink, self.out,
                   self.lse, stream, arrivals=self.arrivals)
                return self.out, self.lse
            fn(*head, self.n_splits, self.sel, self.sel_count, acc, ml, stream=stream)
        else:
            if self.delta is None:
                ops.ps_select_topk(g, self.scores, seq_lens, self.budget, self.n_sink,
                                   self.n_local, self.sel, self.sel_count, stream)
            else:
                ops.ps_select_topdelta(g, q, k_pool, page_table, seq_lens, self.scores,
                                       self.budget, self.n_sink, self.n_local, self.scale,
                                       self.delta, self.sel, self.sel_count, stream)
            ops.ps_sparse_decode(g, q, k_pool, v_pool, page_table, seq_lens, self.sel,
                                 self.sel_count, self.budget, self.scale, self.n_splits, acc, ml,
                                 stream)
        ops.ps_combine(g, acc, ml, self.n_splits, sink, self.out, self.lse, stream)
        return self.out, self.lse

    def dense(self, q, k_pool, v_pool, page_table, seq_lens, sink=None, stream=None):
        g = self.g
        acc, ml = self.partials(self.dense_splits)
        ops.ps_full_decode(g, q, k_pool, v_pool, page_table, seq_lens, self.scale,
                           self.dense_splits, acc, ml, stream)
        ops.ps_combine(g, acc, ml, self.dense_splits, sink, self.out, self.lse, stream)
        return self.out, self.lse

    def __call__(self, q, k_pool, v_pool, meta, page_table, seq_lens, seq_lens_host, sink=None,
                 stream=None):
        """Run the step; returns (out, lse, path)."""
        path = self.path_for(seq_lens_host)
        if path == "dense":
            out, lse = self.dense(q, k_pool, v_pool, page_table, seq_lens, sink, stream)
        else:
            out, lse = self.sparse(q, k_pool, v_pool, meta, page_table, seq_lens, sink, stream)
        return out, lse, path


def build_meta(geom: Geometry, k_pool, page_table, seq_lens, stream=None) -> torch.Tensor:
    """Allocate and fill the metadata of every page of every request (per
    physical page or per logical slot, as geom.meta_layout says)."""
    meta = torch.empty(ops.meta_shape(geom), device=k_pool.device, dtype=geom.meta_dtype)
    ops.ps_build_page_meta(geom, k_pool, page_table, seq_lens, None, geom.max_pages, meta, stream)
    return meta
