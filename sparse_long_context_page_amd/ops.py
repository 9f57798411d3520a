"""Python binding of the C ABI: one function per entry point, same names.

Argument marshalling only. Each function checks that the torch tensors it is
given have the layout the header documents (device, dtype, shape,
contiguity), passes their device pointers and the current HIP stream to the
library, and raises PsError on a non-zero status. Every step of the method
runs in the library's HIP kernels; nothing here computes.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

from . import _lib

KV_DTYPES = {torch.bfloat16: _lib.PS_BF16, torch.float32: _lib.PS_F32}
META_FORMATS = {"kv": _lib.PS_META_KV, "fp8": _lib.PS_META_FP8_E4M3}
META_LAYOUTS = {"physical": _lib.PS_META_PHYSICAL, "logical": _lib.PS_META_LOGICAL}


@dataclasses.dataclass(frozen=True)
class Geometry:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_pages: int
    num_phys_pages: int
    kv_dtype: torch.dtype = torch.bfloat16
    page_size: int = 16
    meta_format: str = "kv"  # "kv": metadata in kv_dtype; "fp8": 8-bit E4M3 bounds
    # "physical": metadata per physical page [P_phys, Hkv, 2, D];
    # "logical": per request in logical page order [B, Hkv, max_pages, 2, D]
    meta_layout: str = "physical"

    @property
    def meta_dtype(self) -> torch.dtype:
        """torch dtype of the metadata pool (uint8 codes for "fp8")."""
        return torch.uint8 if self.meta_format == "fp8" else self.kv_dtype

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def c(self) -> _lib.PsGeom:
        if self.kv_dtype not in KV_DTYPES:
            raise TypeError(f"unsupported kv dtype {self.kv_dtype}")
        if self.meta_format not in META_FORMATS:
            raise ValueError(f"unknown metadata format {self.meta_format!r}")
        if self.meta_layout not in META_LAYOUTS:
            raise ValueError(f"unknown metadata layout {self.meta_layout!r}")
        return _lib.PsGeom(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                           self.page_size, self.max_pages, self.num_phys_pages,
                           KV_DTYPES[self.kv_dtype], META_FORMATS[self.meta_format],
                           META_LAYOUTS[self.meta_layout])

    @staticmethod
    def of(q: torch.Tensor, k_pool: torch.Tensor, page_table: torch.Tensor,
           meta_format: str = "kv", meta_layout: str = "physical") -> "Geometry":
        b, hq, d = q.shape
        p_phys, hkv, ps, d2 = k_pool.shape
        if d2 != d or page_table.shape[0] != b:
            raise ValueError("q, k_pool and page_table disagree on batch or head_dim")
        return Geometry(b, hq, hkv, d, page_table.shape[1], p_phys, k_pool.dtype, ps, meta_format,
                        meta_layout)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _pool_shape(g: Geometry):
    return (g.num_phys_pages, g.num_kv_heads, g.page_size, g.head_dim)


def meta_shape(g: Geometry):
    if g.meta_layout == "logical":
        return (g.batch, g.num_kv_heads, g.max_pages, 2, g.head_dim)
    return (g.num_phys_pages, g.num_kv_heads, 2, g.head_dim)


def ps_build_page_meta(g: Geometry, k_pool, page_table, seq_lens, page_begin, n_pages: int, meta,
                       stream=None) -> None:
    lib = _lib.load()
    rc = lib.ps_build_page_meta(
        g.c(), _ptr(k_pool, "k_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)),
        _ptr(page_begin, "page_begin", torch.int32, (g.batch,), optional=True), int(n_pages),
        _ptr(meta, "meta", g.meta_dtype, meta_shape(g)), _stream(stream))
    _lib.check("ps_build_page_meta", rc)


def ps_score_pages(g: Geometry, q, meta, page_table, seq_lens, scores, stream=None) -> None:
    lib = _lib.load()
    rc = lib.ps_score_pages(
        g.c(), _ptr(q, "q", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(meta, "meta", g.meta_dtype, meta_shape(g)),
        _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)),
        _ptr(scores, "scores", torch.float32, (g.batch, g.num_kv_heads, g.max_pages)),
        _stream(stream))
    _lib.check("ps_score_pages", rc)


def ps_refresh_score_pages(g: Geometry, q, k_pool, meta, page_table, seq_lens, scores,
                           stream=None) -> None:
    """ps_build_page_meta of each request's last page, then ps_score_pages,
    in one launch (bf16 pools)."""
    lib = _lib.load()
    rc = lib.ps_refresh_score_pages(
        g.c(), _ptr(q, "q", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(k_pool, "k_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(meta, "meta", g.meta_dtype, meta_shape(g)),
        _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)),
        _ptr(scores, "scores", torch.float32, (g.batch, g.num_kv_heads, g.max_pages)),
        _stream(stream))
    _lib.check("ps_refresh_score_pages", rc)


def ps_select_topk(g: Geometry, scores, seq_lens, budget_pages: int, n_sink_pages: int,
                   n_local_pages: int, sel, sel_count, stream=None) -> None:
    lib = _lib.load()
    rc = lib.ps_select_topk(
        g.c(), _ptr(scores, "scores", torch.float32, (g.batch, g.num_kv_heads, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)), int(budget_pages),
        int(n_sink_pages), int(n_local_pages),
        _ptr(sel, "sel", torch.int32, (g.batch, g.num_kv_heads, budget_pages)),
        _ptr(sel_count, "sel_count", torch.int32, (g.batch, g.num_kv_heads)), _stream(stream))
    _lib.check("ps_select_topk", rc)


def ps_select_topdelta(g: Geometry, q, k_pool, page_table, seq_lens, scores, budget_pages: int,
                       n_sink_pages: int, n_local_pages: int, scale: float, delta: float, sel,
                       sel_count, stream=None) -> None:
    """Top-delta selection: forced pages plus the best pages whose scaled
    score reaches the smallest pseudo-max of the group minus delta, at most
    budget_pages in all."""
    lib = _lib.load()
    rc = lib.ps_select_topdelta(
        g.c(), _ptr(q, "q", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(k_pool, "k_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)),
        _ptr(scores, "scores", torch.float32, (g.batch, g.num_kv_heads, g.max_pages)),
        int(budget_pages), int(n_sink_pages), int(n_local_pages), float(scale), float(delta),
        _ptr(sel, "sel", torch.int32, (g.batch, g.num_kv_heads, budget_pages)),
        _ptr(sel_count, "sel_count", torch.int32, (g.batch, g.num_kv_heads)), _stream(stream))
    _lib.check("ps_select_topdelta", rc)


def ps_sparse_decode(g: Geometry, q, k_pool, v_pool, page_table, seq_lens, sel, sel_count,
                     budget_pages: int, scale: float, n_splits: int, part_acc, part_ml,
                     stream=None) -> None:
    lib = _lib.load()
    rc = lib.ps_sparse_decode(
        g.c(), _ptr(q, "q", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(k_pool, "k_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(v_pool, "v_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)),
        _ptr(sel, "sel", torch.int32, (g.batch, g.num_kv_heads, budget_pages)),
        _ptr(sel_count, "sel_count", torch.int32, (g.batch, g.num_kv_heads)), int(budget_pages),
        float(scale), int(n_splits),
        _ptr(part_acc, "part_acc", torch.float32, (g.batch, g.num_q_heads, n_splits, g.head_dim)),
        _ptr(part_ml, "part_ml", torch.float32, (g.batch, g.num_q_heads, n_splits, 2)),
        _stream(stream))
    _lib.check("ps_sparse_decode", rc)


# Limits of the fused selection + decode (the unfused entry points have none
# of these): bf16 pools, at most 8192 pages per request and 512 list slots
# per split.
SELECT_DECODE_MAX_PAGES = 8192
SELECT_DECODE_MAX_SPLIT_PAGES = 512


def select_decode_supported(g: Geometry, budget_pages: int, n_splits: int) -> bool:
    return (g.max_pages <= SELECT_DECODE_MAX_PAGES
            and -(-budget_pages // n_splits) <= SELECT_DECODE_MAX_SPLIT_PAGES)


def _select_decode_args(g: Geometry, q, k_pool, v_pool, page_table, seq_lens, scores,
                        budget_pages: int, n_sink: int, n_local: int, scale: float):
    return (g.c(), _ptr(q, "q", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
            _ptr(k_pool, "k_pool", g.kv_dtype, _pool_shape(g)),
            _ptr(v_pool, "v_pool", g.kv_dtype, _pool_shape(g)),
            _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
            _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)),
            _ptr(scores, "scores", torch.float32, (g.batch, g.num_kv_heads, g.max_pages)),
            int(budget_pages), int(n_sink), int(n_local), float(scale))


def _select_decode_outputs(g: Geometry, budget_pages: int, ns: int, sel, sel_count, part_acc,
                           part_ml, sink, out, lse, arrivals, stream):
    return (_ptr(sel, "sel", torch.int32, (g.batch, g.num_kv_heads, budget_pages),
                 optional=True),
            _ptr(sel_count, "sel_count", torch.int32, (g.batch, g.num_kv_heads), optional=True),
            _ptr(part_acc, "part_acc", torch.float32, (g.batch, g.num_q_heads, ns, g.head_dim),
                 optional=True),
            _ptr(part_ml, "part_ml", torch.float32, (g.batch, g.num_q_heads, ns, 2),
                 optional=True),
            _ptr(sink, "sink", torch.float32, (g.num_q_heads,), optional=True),
            _ptr(out, "out", torch.float32, (g.batch, g.num_q_heads, g.head_dim), optional=True),
            _ptr(lse, "lse", torch.float32, (g.batch, g.num_q_heads), optional=True),
            _ptr(arrivals, "arrivals", torch.int32, (g.batch, g.num_kv_heads), optional=True),
            _stream(stream))


def ps_select_sparse_decode(g: Geometry, q, k_pool, v_pool, page_table, seq_lens, scores,
                            budget_pages: int, n_sink: int, n_local: int, scale: float,
                            n_splits: int, sel, sel_count, part_acc, part_ml, sink=None,
                            out=None, lse=None, stream=None, arrivals=None) -> None:
    """ps_select_topk and ps_sparse_decode in one launch (sel and sel_count
    may both be None); with out also the merge of ps_combine (with more than
    one split: arrivals, [B, Hkv] int32 on the device, zero before and after)."""
    lib = _lib.load()
    ns = int(n_splits)
    rc = lib.ps_select_sparse_decode(
        *_select_decode_args(g, q, k_pool, v_pool, page_table, seq_lens, scores, budget_pages,
                             n_sink, n_local, scale), ns,
        *_select_decode_outputs(g, budget_pages, ns, sel, sel_count, part_acc, part_ml, sink,
                                out, lse, arrivals, stream))
    _lib.check("ps_select_sparse_decode", rc)


def ps_select_sparse_decode_noalloc(g: Geometry, q, k_pool, v_pool, page_table, seq_lens,
                                    scores, budget_pages: int, n_sink: int, n_local: int,
                                    scale: float, n_splits: int, sel, sel_count, sink, out,
                                    lse=None, stream=None) -> None:
    """ps_select_sparse_decode with out, its split partials and arrival
    counters in the library's fixed workspace (nothing allocated; calls that
    overlap on one GPU race)."""
    lib = _lib.load()
    ns = int(n_splits)
    rc = lib.ps_select_sparse_decode_noalloc(
        *_select_decode_args(g, q, k_pool, v_pool, page_table, seq_lens, scores, budget_pages,
                             n_sink, n_local, scale), ns,
        _ptr(sel, "sel", torch.int32, (g.batch, g.num_kv_heads, budget_pages), optional=True),
        _ptr(sel_count, "sel_count", torch.int32, (g.batch, g.num_kv_heads), optional=True),
        _ptr(sink, "sink", torch.float32, (g.num_q_heads,), optional=True),
        _ptr(out, "out", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(lse, "lse", torch.float32, (g.batch, g.num_q_heads), optional=True),
        _stream(stream))
    _lib.check("ps_select_sparse_decode_noalloc", rc)


def ps_select_topdelta_sparse_decode(g: Geometry, q, k_pool, v_pool, page_table, seq_lens,
                                     scores, budget_pages: int, n_sink: int, n_local: int,
                                     scale: float, delta: float, n_splits: int, sel, sel_count,
                                     part_acc, part_ml, sink=None, out=None, lse=None,
                                     stream=None, arrivals=None) -> None:
    """ps_select_topdelta and ps_sparse_decode in one launch (arguments as
    ps_select_sparse_decode, delta as ps_select_topdelta)."""
    lib = _lib.load()
    ns = int(n_splits)
    rc = lib.ps_select_topdelta_sparse_decode(
        *_select_decode_args(g, q, k_pool, v_pool, page_table, seq_lens, scores, budget_pages,
                             n_sink, n_local, scale), float(delta), ns,
        *_select_decode_outputs(g, budget_pages, ns, sel, sel_count, part_acc, part_ml, sink,
                                out, lse, arrivals, stream))
    _lib.check("ps_select_topdelta_sparse_decode", rc)


def ps_full_decode(g: Geometry, q, k_pool, v_pool, page_table, seq_lens, scale: float,
                   n_splits: int, part_acc, part_ml, stream=None) -> None:
    lib = _lib.load()
    rc = lib.ps_full_decode(
        g.c(), _ptr(q, "q", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(k_pool, "k_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(v_pool, "v_pool", g.kv_dtype, _pool_shape(g)),
        _ptr(page_table, "page_table", torch.int32, (g.batch, g.max_pages)),
        _ptr(seq_lens, "seq_lens", torch.int32, (g.batch,)), float(scale), int(n_splits),
        _ptr(part_acc, "part_acc", torch.float32, (g.batch, g.num_q_heads, n_splits, g.head_dim)),
        _ptr(part_ml, "part_ml", torch.float32, (g.batch, g.num_q_heads, n_splits, 2)),
        _stream(stream))
    _lib.check("ps_full_decode", rc)


def ps_combine(g: Geometry, part_acc, part_ml, n_splits: int, sink, out, lse, stream=None) -> None:
    lib = _lib.load()
    rc = lib.ps_combine(
        g.c(),
        _ptr(part_acc, "part_acc", torch.float32, (g.batch, g.num_q_heads, n_splits, g.head_dim)),
        _ptr(part_ml, "part_ml", torch.float32, (g.batch, g.num_q_heads, n_splits, 2)),
        int(n_splits), _ptr(sink, "sink", torch.float32, (g.num_q_heads,), optional=True),
        _ptr(out, "out", torch.float32, (g.batch, g.num_q_heads, g.head_dim)),
        _ptr(lse, "lse", torch.float32, (g.batch, g.num_q_heads), optional=True),
        _stream(stream))
    _lib.check("ps_combine", rc)


def ps_strerror(status: int) -> str:
    return _lib.strerror(status)


def ps_abi_version() -> int:
    return _lib.load().ps_abi_version()


def default_scale(head_dim: int) -> float:
    """1/sqrt(D) as the fp32 value the kernels receive."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))
